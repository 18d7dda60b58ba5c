"""GPU parity of mla_project_append (down-projection of the new tokens' hidden
states to their latent rows and RoPE keys, then the cache append) against the
CPU oracle's kv_down_project / project_append_row."""

import numpy as np
import pytest
import torch

import synth
from helpers import gpu_f64, to_f64
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

D_C, D_R = synth.D_C, synth.D_ROPE
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2}


def oracle_rows(h, w_dkv, w_kr, pos, cache_dtype):
    """Oracle rows [B, 576] (dequantised for fp8) and fp8 scales."""
    act = "f32" if h.dtype == torch.float32 else "bf16"
    hh, wd, wk = to_f64(h, act), to_f64(w_dkv, act), to_f64(w_kr, act)
    rows, scales = [], []
    for b in range(h.shape[0]):
        lat, rope, s, _ = orc.project_append_row(hh[b], wd, wk, int(pos[b]), cache_dtype)
        rows.append(np.concatenate([lat, rope]))
        scales.append(s)
    return np.stack(rows), scales


def cache_values(cache, scales, rows, cache_dtype):
    got = to_f64(cache[rows].cpu(), cache_dtype)
    if cache_dtype == "fp8":
        got = got * to_f64(scales[rows].cpu(), "bf16")[:, None]
    return got


def check_rows(got, ref, cache_dtype):
    """Row-relative max error (each row against its own largest value)."""
    err = np.max(np.abs(got - ref), axis=1) / np.max(np.abs(ref), axis=1)
    worst = float(err.max())
    print(f"[result] worst row error {worst:.3e} (tolerance {TOL[cache_dtype]})", flush=True)
    assert worst <= TOL[cache_dtype], worst


@pytest.mark.parametrize("act,cache_dtype,B,d_model", [
    ("bf16", "bf16", 37, 7168),     # DeepSeek-V3 width, ragged batch (two 32-row tiles)
    ("bf16", "bf16", 128, 7168),    # four 32-row tiles
    ("bf16", "fp8", 64, 7168),      # the fp8 cache
    ("bf16", "bf16", 200, 1024),    # two batch groups of 128, ragged
    ("bf16", "bf16", 1, 64),        # a single 64-wide chunk
    ("f32", "f32", 3, 512),         # fp32 operands and cache
    ("f32", "bf16", 33, 2048),      # fp32 operands, bf16 cache, 33 rows
    ("f32", "fp8", 5, 512),         # fp32 operands, fp8 cache (two launches)
    ("bf16", "bf16", 1000, 1024),   # eight batch groups of 128, the last ragged
])
def test_project_append_contiguous(gpu, act, cache_dtype, B, d_model):
    cap = 8
    print(f"[case] project_append act={act} cache={cache_dtype} B={B} d_model={d_model}",
          flush=True)
    h, w_dkv, w_kr = synth.projection_inputs(40 + B, B, act, d_model)
    pos = torch.randint(0, cap, (B,), generator=torch.Generator().manual_seed(B),
                        dtype=torch.int32)
    rows = B * cap
    fp8 = cache_dtype == "fp8"
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[cache_dtype]
    cache0 = torch.full((rows, 576), 3, dtype=dt)
    scales0 = torch.full((rows,), 0.5, dtype=torch.bfloat16) if fp8 else None
    cache = cache0.cuda()
    scales = scales0.cuda() if fp8 else None
    lat, rope = gpu.split_cache(cache)
    gpu.project_append(h.cuda(), w_dkv.cuda(), w_kr.cuda(), pos.cuda(), lat, rope, heads=128,
                       scales=scales, seq_capacity=cap)
    torch.cuda.synchronize()
    written = [b * cap + int(pos[b]) for b in range(B)]
    ref, ref_scales = oracle_rows(h, w_dkv, w_kr, pos, cache_dtype)
    check_rows(cache_values(cache, scales, written, cache_dtype), ref, cache_dtype)
    if fp8:
        got_s = to_f64(scales.cpu()[written], "bf16")
        assert np.max(np.abs(got_s / np.array(ref_scales) - 1)) <= 2 ** -7
    others = sorted(set(range(rows)) - set(written))
    assert torch.equal(cache.cpu()[others], cache0[others])


def test_project_append_paged_and_repeatable(gpu):
    """Paged slots; two calls on the same inputs write the same bytes (the
    partial sums are added in a fixed order)."""
    B, bs = 5, 64
    h, w_dkv, w_kr = synth.projection_inputs(77, B, "bf16")
    table = torch.tensor([[3, 0], [1, 7], [6, 2], [4, 8], [9, 5]], dtype=torch.int32)
    pos = torch.tensor([0, 64, 127, 5, 100], dtype=torch.int32)
    rows = [orc.paged_row(table.numpy(), b, int(pos[b]), bs) for b in range(B)]
    assert rows == [3 * 64, 7 * 64, 2 * 64 + 63, 4 * 64 + 5, 5 * 64 + 36]
    outs = []
    for _ in range(2):
        cache = torch.zeros((10 * bs, 576), dtype=torch.bfloat16, device="cuda")
        lat, rope = gpu.split_cache(cache)
        gpu.project_append(h.cuda(), w_dkv.cuda(), w_kr.cuda(), pos.cuda(), lat, rope,
                           heads=128, block_table=table.cuda(), block_size=bs)
        torch.cuda.synchronize()
        outs.append(cache.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref, _ = oracle_rows(h, w_dkv, w_kr, pos, "bf16")
    check_rows(to_f64(outs[0][rows], "bf16"), ref, "bf16")
    others = sorted(set(range(10 * bs)) - set(rows))
    assert not outs[0][others].view(torch.int16).any()


def test_projected_token_then_decode(gpu):
    """The new token computes only its own cache row, then reads the whole
    history ("How DeepSeek Rewrote the Transformer [MLA]", section "Classic
    attention and the cost of the KV cache"): project + append the token at
    position n-1 of every sequence, decode over n rows, and compare with the
    oracle's decode over the oracle's own rows for that token."""
    B, N, H = 4, 300, 128
    lengths = torch.tensor([N, 117, 1, 256], dtype=torch.int32)
    inp = synth.make_inputs(2, B=B, N=N, lengths=lengths).to("cuda")
    h, w_dkv, w_kr = synth.projection_inputs(91, B, "bf16")
    pos = (inp.lengths - 1).contiguous()
    lat, rope = gpu.split_cache(inp.cache)
    gpu.project_append(h.cuda(), w_dkv.cuda(), w_kr.cuda(), pos, lat, rope, heads=H,
                       seq_capacity=inp.seq_capacity)
    out, _ = gpu.decode_inputs(inp)
    torch.cuda.synchronize()
    # oracle: the cache's earlier rows as the GPU holds them, the new row from
    # the oracle's projection (not from the GPU's)
    cpu = inp.to("cpu")
    ref_rows, _ = oracle_rows(h, w_dkv, w_kr, pos.cpu(), "bf16")
    kind = "bf16"
    qn, qp = to_f64(cpu.q_nope, kind), to_f64(cpu.q_pe, kind)
    wuk, wuv = to_f64(cpu.w_uk, kind), to_f64(cpu.w_uv, kind)
    lat_l, rope_l = [], []
    for b in range(B):
        n = int(lengths[b])
        rows = orc.gather_rows(b, n, seq_capacity=cpu.seq_capacity)
        vals = to_f64(cpu.cache[torch.from_numpy(rows)], "bf16")
        vals[n - 1] = ref_rows[b]
        lat_l.append(vals[:, :D_C])
        rope_l.append(vals[:, D_C:])
    ref, _ = orc.decode(qn, qp, wuk, wuv, lat_l, rope_l, cpu.scale)
    got = gpu_f64(out)
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    print(f"[result] decode after projected append: {err:.3e}", flush=True)
    assert err <= 1e-2


def test_workspace_reused_across_calls(gpu):
    """One workspace serves calls of different batch sizes and cache types in
    a row (its contents on entry do not matter): every call's rows match the
    oracle."""
    D = 2048
    cases = [(64, "bf16"), (200, "bf16"), (3, "f32"), (130, "fp8"), (64, "bf16")]
    ws = torch.full((max(gpu.project_workspace_size(B, D) for B, _ in cases),), 0x5A,
                    dtype=torch.uint8, device="cuda")
    for i, (B, cache_dtype) in enumerate(cases):
        print(f"[case] reused workspace call {i}: B={B} cache={cache_dtype}", flush=True)
        h, w_dkv, w_kr = synth.projection_inputs(300 + i, B, "bf16", D)
        pos = torch.full((B,), 2, dtype=torch.int32)
        fp8 = cache_dtype == "fp8"
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[cache_dtype]
        cache = torch.zeros((B * 4, 576), dtype=dt, device="cuda")
        scales = torch.ones(B * 4, dtype=torch.bfloat16, device="cuda") if fp8 else None
        lat, rope = gpu.split_cache(cache)
        gpu.project_append(h.cuda(), w_dkv.cuda(), w_kr.cuda(), pos.cuda(), lat, rope,
                           heads=128, scales=scales, seq_capacity=4, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = oracle_rows(h, w_dkv, w_kr, pos, cache_dtype)
        rows = [b * 4 + 2 for b in range(B)]
        check_rows(cache_values(cache, scales, rows, cache_dtype), ref, cache_dtype)


def test_project_append_paged_fp8(gpu):
    """fp8 cache through a block table (the two-launch form: whole-row
    scale), rows in three different blocks, against the oracle's rows."""
    B, bs = 3, 32
    h, w_dkv, w_kr = synth.projection_inputs(55, B, "bf16")
    table = torch.tensor([[4, 1], [0, 5], [2, 3]], dtype=torch.int32)
    pos = torch.tensor([33, 0, 63], dtype=torch.int32)
    rows = [orc.paged_row(table.numpy(), b, int(pos[b]), bs) for b in range(B)]
    assert rows == [32 + 1, 0, 3 * 32 + 31]
    cache = torch.zeros((6 * bs, 576), dtype=torch.uint8, device="cuda")
    scales = torch.ones(6 * bs, dtype=torch.bfloat16, device="cuda")
    lat, rope = gpu.split_cache(cache)
    gpu.project_append(h.cuda(), w_dkv.cuda(), w_kr.cuda(), pos.cuda(), lat, rope, heads=128,
                       scales=scales, block_table=table.cuda(), block_size=bs)
    torch.cuda.synchronize()
    ref, ref_scales = oracle_rows(h, w_dkv, w_kr, pos, "fp8")
    check_rows(cache_values(cache, scales, rows, "fp8"), ref, "fp8")
    got_s = to_f64(scales.cpu()[rows], "bf16")
    assert np.max(np.abs(got_s / np.array(ref_scales) - 1)) <= 2 ** -7
    others = sorted(set(range(6 * bs)) - set(rows))
    assert not cache.cpu()[others].any()


@pytest.mark.parametrize("cfg,cache_dtype", [(3, "bf16"), (2, "fp8"), (1, "f32")])
def test_decode_append_from_projection_equals_two_calls(gpu, cfg, cache_dtype):
    """mla_project, then a decode call whose append takes the projection's
    workspace (mla_append_args.projected), writes the same cache bytes and
    returns the same output and lse bits as mla_project_append followed by
    a decode without append (the partial sums are added in the same order)."""
    import dataclasses
    B, N, D = 4, 300, 2048
    lengths = torch.tensor([N, 200, 1, 64][:B], dtype=torch.int32)
    inp = synth.make_inputs(cfg, B=B, N=N, lengths=lengths, cache_dtype=cache_dtype,
                            paged=(cfg == 3)).to("cuda")
    act = "f32" if cache_dtype == "f32" else "bf16"
    h, w_dkv, w_kr = [t.cuda() for t in synth.projection_inputs(66, B, act, D)]
    pos = (inp.lengths - 1).contiguous()
    print(f"[case] projected append in decode cfg={cfg} cache={cache_dtype} act={act}", flush=True)

    def fresh():
        return dataclasses.replace(inp, cache=inp.cache.clone(),
                                   scales=None if inp.scales is None else inp.scales.clone())

    two = fresh()
    lat, rope = gpu.split_cache(two.cache)
    gpu.project_append(h, w_dkv, w_kr, pos, lat, rope, heads=inp.H, scales=two.scales,
                       seq_capacity=inp.seq_capacity, block_table=inp.block_table,
                       block_size=inp.block_size)
    out_a, lse_a = gpu.decode_inputs(two)
    one = fresh()
    ws = torch.empty(gpu.project_workspace_size(B, D), dtype=torch.uint8, device="cuda")
    gpu.project(h, w_dkv, w_kr, ws, heads=inp.H)
    out_b, lse_b = gpu.decode_inputs(one, append=(None, None, pos, 10000.0, ws, D))
    torch.cuda.synchronize()
    assert not torch.equal(two.cache.view(torch.uint8), inp.cache.view(torch.uint8))
    assert torch.equal(two.cache.view(torch.uint8), one.cache.view(torch.uint8))
    if two.scales is not None:
        assert torch.equal(two.scales, one.scales)
    assert torch.equal(out_a.view(torch.uint8), out_b.view(torch.uint8))
    assert torch.equal(lse_a, lse_b)
