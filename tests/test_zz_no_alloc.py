"""The allocation-free decode entry point (mla_decode_paged_noalloc) against
mla_decode_paged with a workspace: the same kernels with the same split
plan, so outputs, lse and appended cache rows are bit-identical. Two calls
in a row, the second with a smaller input (the scratch keeps the first
call's contents), for a bf16 and an fp8 cache, one of them appending."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def compare(gpu, cfg, B, N, lengths, cache_dtype=None, append=False, seed=0):
    print(f"[case] noalloc cfg={cfg} B={B} N={N} cache={cache_dtype} append={append}", flush=True)
    inp = synth.make_inputs(cfg, B=B, N=N, lengths=lengths, paged=True, cache_dtype=cache_dtype)
    dev = inp.to("cuda")
    cache_ref = dev.cache.clone()
    scales_ref = None if dev.scales is None else dev.scales.clone()
    app = None
    if append:
        c_new, k_new = synth.append_inputs(8100 + seed, B, "bf16", device="cuda")
        app = (c_new, k_new, (inp.lengths - 1).to("cuda"))
    kw = dict(block_table=dev.block_table, block_size=dev.block_size,
              softmax_scale=dev.scale, append=app)
    lat, rope = gpu.split_cache(cache_ref)
    ref_out, ref_lse = gpu.decode_paged(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, lat, rope,
                                        dev.lengths, dev.max_len, scales=scales_ref, **kw)
    lat, rope = gpu.split_cache(dev.cache)
    out, lse = gpu.decode_paged_noalloc(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, lat, rope,
                                        dev.lengths, dev.max_len, scales=dev.scales, **kw)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref_out))
    assert torch.equal(bits(lse), bits(ref_lse))
    assert torch.equal(dev.cache.view(torch.uint8), cache_ref.view(torch.uint8))
    if scales_ref is not None:
        assert torch.equal(bits(dev.scales), bits(scales_ref))
    print(f"[result] bit-identical out {tuple(out.shape)} and lse", flush=True)


def test_noalloc_bf16_then_smaller(gpu):
    compare(gpu, 3, 48, 2048, torch.randint(1, 2049, (48,), generator=torch.Generator().manual_seed(1)))
    compare(gpu, 3, 3, 300, torch.tensor([300, 1, 77], dtype=torch.int32), append=True, seed=1)


def test_noalloc_fp8_then_smaller(gpu):
    compare(gpu, 5, 8, 4096, torch.full((8,), 4096, dtype=torch.int32), cache_dtype="fp8",
            append=True, seed=2)
    compare(gpu, 5, 2, 100, torch.tensor([100, 33], dtype=torch.int32), cache_dtype="fp8")


def test_noalloc_full_benchmark_size(gpu):
    """The benchmark's workload (B=64, N=4096, paged bf16) fits the scratch."""
    compare(gpu, "3u", 64, 4096, torch.full((64,), 4096, dtype=torch.int32), append=True, seed=3)


def test_noalloc_length_aware_matches_workspace_call(gpu):
    """mla_decode_paged_noalloc with the length-aware plan (its items and
    split counts in the library's scratch) gives the bits of the call with a
    workspace."""
    lengths = torch.tensor([3000, 64, 1200, 5, 2999], dtype=torch.int32)
    inp = synth.make_inputs(3, B=5, N=3000, lengths=lengths, paged=True).to("cuda")
    print("[case] length-aware noalloc vs workspace", flush=True)
    a_out, a_lse = gpu.decode_inputs(inp, length_aware=True)
    lat, rope = gpu.split_cache(inp.cache)
    b_out, b_lse = gpu.decode_paged_noalloc(inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, lat, rope,
                                            inp.lengths, inp.max_len,
                                            block_table=inp.block_table,
                                            block_size=inp.block_size, softmax_scale=inp.scale,
                                            length_aware=True)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.uint8), b_out.view(torch.uint8))
    assert torch.equal(a_lse, b_lse)
