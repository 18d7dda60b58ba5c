"""The decode and prefill entry points under HIP graph capture (through
torch.cuda.CUDAGraph on the caller's stream): the launches take only
caller-owned buffers (workspace, outputs) or the library's static scratch,
record no memset and allocate nothing, so a captured call replays the same
kernels. Each case captures one call, then replays it three times with the
program's own eager work (another decode into the same workspace, fills of
the outputs) and synchronizations between the replays, and checks every
replay against the eager result of the same call bit for bit (the kernels
are deterministic). Also: a decode call marshalled once and re-issued (the
benchmark's loop) against the direct call."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def capture_and_replay(call, outputs, between):
    """call(): the captured work, writing into `outputs`; between(): eager
    work run before each replay."""
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # the capture recipe: a warm-up on a side stream
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for o in outputs:
            o.zero_()
        between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(bits(o), bits(r)), f"replay {rep} differs"
        print(f"[result] replay {rep}: bit-identical", flush=True)


def decode_case(gpu, cfg, B, N, lengths, paged, cache_dtype=None, num_splits=0, append=False,
                seed=0, length_aware=False, other_lengths=None):
    print(f"[case] graph decode cfg={cfg} B={B} N={N} paged={paged} cache={cache_dtype} "
          f"splits={num_splits} append={append} length_aware={length_aware}", flush=True)
    inp = synth.make_inputs(cfg, B=B, N=N, lengths=lengths, paged=paged,
                            cache_dtype=cache_dtype).to("cuda")
    other = synth.make_inputs(cfg, B=B, N=N,
                              lengths=lengths if other_lengths is None else other_lengths,
                              paged=paged, cache_dtype=cache_dtype, layer=1).to("cuda")
    act, cdt = gpu.dtype_code(inp.q_nope.dtype), gpu.dtype_code(inp.cache.dtype)
    ws = torch.empty(gpu.workspace_size(inp.H, B, max(inp.max_len, other.max_len), act, cdt,
                                        num_splits, length_aware),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, inp.H, 128), dtype=inp.q_nope.dtype, device="cuda")
    lse = torch.empty((B, inp.H), dtype=torch.float32, device="cuda")
    app = None
    if append:
        c_new, k_new = synth.append_inputs(8200 + seed, B, "bf16", device="cuda")
        app = (c_new, k_new, (inp.lengths - 1).to("cuda"))

    def call():
        gpu.decode_inputs(inp, out=out, lse=lse, workspace=ws, num_splits=num_splits, append=app,
                          length_aware=length_aware)

    call()
    torch.cuda.synchronize()
    capture_and_replay(call, [out, lse],
                       lambda: gpu.decode_inputs(other, workspace=ws, num_splits=num_splits,
                                                 length_aware=length_aware))


def test_graph_decode_bf16_paged_append(gpu):
    """bf16, paged, ragged lengths, the new rows appended in the same call."""
    lengths = torch.tensor([1000, 1, 300, 777, 64, 65, 999, 512], dtype=torch.int32)
    decode_case(gpu, 3, 8, 1000, lengths, paged=True, append=True, seed=1)


def test_graph_decode_length_aware(gpu):
    """The length-aware plan (made in the absorb launch, in the workspace):
    between replays an eager call plans other lengths into the same
    workspace, and every replay re-plans its own."""
    lengths = torch.tensor([1000, 1, 300, 777, 64, 65, 999, 512], dtype=torch.int32)
    other = torch.tensor([40, 1000, 1000, 3, 700, 999, 2, 1000], dtype=torch.int32)
    decode_case(gpu, 3, 8, 1000, lengths, paged=True, append=True, seed=4, length_aware=True,
                other_lengths=other)


def test_graph_decode_two_level_merge(gpu):
    """70 splits: the two-level merge and the column-split final merge."""
    lengths = torch.tensor([2240, 1540, 33], dtype=torch.int32)
    decode_case(gpu, 2, 3, 2240, lengths, paged=False, num_splits=70, seed=2)


def test_graph_decode_fp8(gpu):
    """fp8 cache on the fp8 matrix cores."""
    lengths = torch.tensor([700, 300, 64, 1], dtype=torch.int32)
    decode_case(gpu, 5, 4, 700, lengths, paged=False, cache_dtype="fp8", seed=3)


def test_graph_decode_noalloc(gpu):
    """The allocation-free entry point (the library's static scratch)."""
    print("[case] graph decode noalloc B=6 N=900 paged", flush=True)
    lengths = torch.tensor([900, 5, 450, 899, 128, 33], dtype=torch.int32)
    inp = synth.make_inputs(3, B=6, N=900, lengths=lengths, paged=True).to("cuda")
    other = synth.make_inputs(3, B=6, N=900, lengths=lengths, paged=True, layer=1).to("cuda")
    out = torch.empty((6, inp.H, 128), dtype=inp.q_nope.dtype, device="cuda")
    lse = torch.empty((6, inp.H), dtype=torch.float32, device="cuda")

    def run(d, o=None, l=None):
        lat, rope = gpu.split_cache(d.cache)
        gpu.decode_paged_noalloc(d.q_nope, d.q_pe, d.w_uk, d.w_uv, lat, rope, d.lengths,
                                 d.max_len, block_table=d.block_table, block_size=d.block_size,
                                 scales=d.scales, softmax_scale=d.scale, out=o, lse=l)

    run(inp, out, lse)
    torch.cuda.synchronize()
    capture_and_replay(lambda: run(inp, out, lse), [out, lse], lambda: run(other))


def test_graph_prefill(gpu):
    """Prefill: W_UV transpose, decompression and causal attention, a chunk
    of 300 queries after contexts of 700 and 0 tokens."""
    print("[case] graph prefill B=2 T=300", flush=True)
    lengths = torch.tensor([1000, 300], dtype=torch.int32)
    inp = synth.make_inputs(2, B=2, N=1000, lengths=lengths).to("cuda")
    qn, qp = synth.prefill_queries(6300, 2, 300, inp.H, device="cuda")
    qn2, qp2 = synth.prefill_queries(6301, 2, 300, inp.H, device="cuda")
    lat, rope = gpu.split_cache(inp.cache)
    ws = torch.empty(gpu.prefill_workspace_size(inp.H, 2, 1000), dtype=torch.uint8, device="cuda")
    out = torch.empty((2, 300, inp.H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 300, inp.H), dtype=torch.float32, device="cuda")

    def run(q, p, o=None, l=None):
        gpu.prefill(q, p, inp.w_uk, inp.w_uv, lat, rope, inp.lengths, 1000,
                    seq_capacity=inp.seq_capacity, out=o, lse=l, workspace=ws)

    run(qn, qp, out, lse)
    torch.cuda.synchronize()
    capture_and_replay(lambda: run(qn, qp, out, lse), [out, lse], lambda: run(qn2, qp2))


@pytest.mark.parametrize("paged", [True, False])
def test_prepared_decode_matches_direct_call(gpu, paged):
    """A decode call marshalled once (prepare_decode, as the benchmark loop
    issues it) gives the direct call's outputs bit for bit, on every run,
    with and without timing events."""
    print(f"[case] prepared decode paged={paged}", flush=True)
    lengths = torch.tensor([700, 1, 333, 512], dtype=torch.int32)
    inp = synth.make_inputs(3, B=4, N=700, lengths=lengths, paged=paged).to("cuda")
    act, cdt = gpu.dtype_code(inp.q_nope.dtype), gpu.dtype_code(inp.cache.dtype)
    ws = torch.empty(gpu.workspace_size(inp.H, 4, inp.max_len, act, cdt), dtype=torch.uint8,
                     device="cuda")
    c_new, k_new = synth.append_inputs(8300, 4, "bf16", device="cuda")
    app = (c_new, k_new, (inp.lengths - 1).to("cuda"))
    ref_out, ref_lse = gpu.decode_inputs(inp, workspace=ws, append=app)
    torch.cuda.synchronize()
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    call = gpu.prepare_decode_inputs(inp, out=out, lse=lse, workspace=ws, append=app)
    import bench
    ev = bench.HipEvents()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        pair = (ev.create(), ev.create()) if rep == 1 else None
        call.run(pair)
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref_out)) and torch.equal(bits(lse), bits(ref_lse))
        if pair:
            assert ev.elapsed_ms(*pair) > 0.0
            ev.destroy(pair[0])
            ev.destroy(pair[1])
    print("[result] bit-identical on every run", flush=True)
    # the prepared call captured in a graph (run on the capture stream)
    other = synth.make_inputs(3, B=4, N=700, lengths=lengths, paged=paged, layer=1).to("cuda")
    capture_and_replay(lambda: call.run(stream=torch.cuda.current_stream().cuda_stream),
                       [out, lse], lambda: gpu.decode_inputs(other, workspace=ws))
