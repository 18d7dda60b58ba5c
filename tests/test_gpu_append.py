"""GPU parity of mla_cache_append (RoPE on the decoupled key, fp8 row
quantisation, contiguous and paged slots) and of the decode loop built on it
(append one token, decode, repeat), against the CPU oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from helpers import gpu_f64, rel_err_rows, to_f64
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

D_C, D_R = synth.D_C, synth.D_ROPE


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> int:
    """Distance in representable bf16 steps (same-sign values)."""
    a = a_bits.astype(np.int64)
    b = b_bits.astype(np.int64)
    sa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    sb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return int(np.abs(sa - sb).max())


def make_cache(rows, cache_dtype, fill=3):
    if cache_dtype == "fp8":
        cache = torch.full((rows, 576), fill, dtype=torch.uint8)
        scales = torch.full((rows,), 0.5, dtype=torch.bfloat16)
        return cache, scales
    dt = torch.float32 if cache_dtype == "f32" else torch.bfloat16
    return torch.full((rows, 576), float(fill), dtype=dt), None


def run_append(gpu, c, k, pos, cache, scales, **kw):
    dev_cache = cache.cuda()
    dev_scales = None if scales is None else scales.cuda()
    lat, rope = gpu.split_cache(dev_cache)
    print(f"[case] append B={c.shape[0]} in={c.dtype} cache={cache.dtype} pos={pos.tolist()} "
          f"paged={'block_table' in kw}", flush=True)
    bt = kw.pop("block_table", None)
    gpu.cache_append(c.cuda(), k.cuda(), pos.cuda(), lat, rope, heads=128, scales=dev_scales,
                     block_table=None if bt is None else bt.cuda(), **kw)
    torch.cuda.synchronize()
    return dev_cache.cpu(), None if dev_scales is None else dev_scales.cpu()


@pytest.mark.parametrize("in_dtype,cache_dtype", [("bf16", "bf16"), ("f32", "bf16"),
                                                  ("f32", "f32"), ("bf16", "f32")])
def test_append_contiguous(gpu, in_dtype, cache_dtype):
    B, cap = 4, 2048
    pos = torch.tensor([0, 1, 777, 2047], dtype=torch.int32)
    c, k = synth.append_inputs(11, B, in_dtype)
    cache, _ = make_cache(B * cap, cache_dtype)
    out, _ = run_append(gpu, c, k, pos, cache, None, seq_capacity=cap)
    cbits = to_f64(c, in_dtype)
    kbits = to_f64(k, in_dtype)
    written = set()
    for b in range(B):
        row = orc.contiguous_row(b, int(pos[b]), cap)
        written.add(row)
        lat_ref, rope_ref, _, _ = orc.append_row(cbits[b], kbits[b], int(pos[b]), cache_dtype)
        got = to_f64(out[row], cache_dtype)
        # the latent is copied (rounded once when the types differ): exact
        assert np.array_equal(got[:D_C], lat_ref)
        if cache_dtype == "bf16":
            ulps = bf16_ulp_diff(synth.raw_bits(out[row, D_C:]),
                                 orc.bf16_value_to_bits(rope_ref))
            assert ulps <= 1, ulps
        else:
            assert np.allclose(got[D_C:], rope_ref, rtol=2e-7, atol=1e-7)
    # every other row is untouched
    others = [r for r in range(B * cap) if r not in written]
    assert torch.equal(out[others], cache[others])


def test_append_paged(gpu):
    B, bs = 3, 64
    table = torch.tensor([[5, 2, 7], [0, 6, 1], [3, 4, 8]], dtype=torch.int32)
    pos = torch.tensor([70, 0, 191], dtype=torch.int32)
    c, k = synth.append_inputs(12, B, "bf16")
    cache, _ = make_cache(9 * bs, "bf16")
    out, _ = run_append(gpu, c, k, pos, cache, None, block_table=table, block_size=bs)
    rows = [orc.paged_row(table.numpy(), b, int(pos[b]), bs) for b in range(B)]
    assert rows == [2 * 64 + 6, 0, 8 * 64 + 63]
    for b, row in enumerate(rows):
        assert torch.equal(out[row, :D_C].view(torch.int16), c[b].view(torch.int16))
    others = [r for r in range(9 * bs) if r not in rows]
    assert torch.equal(out[others], cache[others])


def test_append_fp8_position0_bit_exact(gpu):
    """At position 0 the rotation is the identity on both sides, so the fp8
    quantiser sees the same fp32 row: scale and every code must match."""
    B = 8
    c, k = synth.append_inputs(13, B, "bf16")
    c[3] = 0                                   # an all-zero latent ...
    k[3] = 0                                   # ... and key: scale 1, codes 0
    c[5, 7] = 1000.0                           # a large value sets the scale
    cache, scales = make_cache(B, "fp8")
    out, sc = run_append(gpu, c, k, torch.zeros(B, dtype=torch.int32), cache, scales,
                         seq_capacity=1)
    for b in range(B):
        _, _, scale, codes = orc.append_row(to_f64(c[b], "bf16"), to_f64(k[b], "bf16"), 0, "fp8")
        assert float(sc[b]) == scale, (b, float(sc[b]), scale)
        assert np.array_equal(out[b].numpy(), codes), b


def test_append_fp8_rotated(gpu):
    """Other positions: the scale within one bf16 step, the dequantised row
    within the fp8 tolerance."""
    B, cap = 4, 40000
    pos = torch.tensor([1, 100, 32767, 39999], dtype=torch.int32)
    c, k = synth.append_inputs(14, B, "f32")
    cache, scales = make_cache(B * cap, "fp8")
    out, sc = run_append(gpu, c, k, pos, cache, scales, seq_capacity=cap)
    for b in range(B):
        row = b * cap + int(pos[b])
        lat, rope, scale, _ = orc.append_row(to_f64(c[b], "f32"), to_f64(k[b], "f32"),
                                             int(pos[b]), "fp8")
        assert bf16_ulp_diff(synth.raw_bits(sc[row:row + 1]),
                             orc.bf16_value_to_bits(np.array([scale]))) <= 1
        deq = orc.e4m3fn_bits_to_f64(out[row].numpy()) * float(sc[row])
        ref = np.concatenate([lat, rope])
        assert np.max(np.abs(deq - ref)) <= 3e-2 * np.max(np.abs(ref))


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_incremental_decode_equals_causal_prefill(gpu, cache_dtype):
    """The KV-cache experiment of the Medium mirror ('From KV Cache to MLA',
    section 'KV Cache'): appending one token at a time and decoding after each
    append gives, at every step t, row t of full causal attention. T=40
    crosses the 32-token tile boundary."""
    B, T, H, cap = 2, 40, 128, 64
    g = torch.Generator().manual_seed(21)
    qn = torch.randn((T, B, H, 128), generator=g).to(torch.bfloat16)
    qp = torch.randn((T, B, H, 64), generator=g).to(torch.bfloat16)
    inp = synth.make_inputs(2, B=B, N=cap, H=H)
    w_uk, w_uv = inp.w_uk, inp.w_uv
    c_all = torch.randn((T, B, D_C), generator=g).to(torch.bfloat16)
    k_all = torch.randn((T, B, D_R), generator=g).to(torch.bfloat16)
    fp8 = cache_dtype == "fp8"
    cache = torch.zeros((B * cap, 576), dtype=torch.uint8 if fp8 else torch.bfloat16).cuda()
    scales = torch.ones(B * cap, dtype=torch.bfloat16).cuda() if fp8 else None
    lat, rope = gpu.split_cache(cache)
    ws = torch.empty(gpu.workspace_size(H, B, cap, gpu.MLA_BF16, gpu.dtype_code(cache.dtype)),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int32, device="cuda")
        gpu.cache_append(c_all[t].cuda(), k_all[t].cuda(), pos, lat, rope, heads=H,
                         scales=scales, seq_capacity=cap)
        out, _ = gpu.decode(qn[t].cuda(), qp[t].cuda(), w_uk.cuda(), w_uv.cuda(), lat, rope,
                            pos + 1, cap, seq_capacity=cap, scales=scales, workspace=ws)
        outs.append(gpu_f64(out))
    torch.cuda.synchronize()
    # oracle: build the cache with its own append, then full causal attention
    wuk, wuv = to_f64(w_uk, "bf16"), to_f64(w_uv, "bf16")
    sc = 1 / np.sqrt(192)
    worst = 0.0
    for b in range(B):
        rows = [orc.append_row(to_f64(c_all[t, b], "bf16"), to_f64(k_all[t, b], "bf16"), t,
                               cache_dtype)[:2] for t in range(T)]
        C = np.stack([r[0] for r in rows])
        R = np.stack([r[1] for r in rows])
        for h in range(0, H, 9):
            full = orc.causal_prefill(to_f64(qn[:, b, h], "bf16"), to_f64(qp[:, b, h], "bf16"),
                                      wuk[h], wuv[h], C, R, sc)
            got = np.stack([outs[t][b, h] for t in range(T)])
            worst = max(worst, rel_err_rows(got, full))
    print(f"[result] incremental decode vs causal prefill: {worst:.3e}", flush=True)
    assert worst <= (3e-2 if fp8 else 1e-2)


@pytest.mark.parametrize("cfg,cache_dtype", [(2, "bf16"), (3, "bf16"), (2, "fp8"), (1, "f32")])
def test_decode_with_append_equals_separate_calls(gpu, cfg, cache_dtype):
    """A decode call given the new rows (mla_decode_options.append) writes the
    cache exactly as mla_cache_append does and returns exactly what the decode
    after that append returns: same cache bytes, same output and lse bits."""
    B = 4 if cfg == 3 else 3
    N = 300
    lengths = torch.tensor([N, N - 37, 1, N - 5][:B], dtype=torch.int32)
    inp = synth.make_inputs(cfg, B=B, N=N, lengths=lengths, cache_dtype=cache_dtype,
                            paged=(cfg == 3)).to("cuda")
    c_new, k_new = synth.append_inputs(5, B, inp.act, device="cuda")
    pos = (inp.lengths - 1).contiguous()
    print(f"[case] decode+append cfg={cfg} cache={cache_dtype} B={B} paged={inp.paged}",
          flush=True)

    def fresh():
        return dataclasses.replace(inp, cache=inp.cache.clone(),
                                   scales=None if inp.scales is None else inp.scales.clone())

    sep = fresh()
    lat, rope = gpu.split_cache(sep.cache)
    gpu.cache_append(c_new, k_new, pos, lat, rope, heads=inp.H, scales=sep.scales,
                     seq_capacity=inp.seq_capacity, block_table=inp.block_table,
                     block_size=inp.block_size)
    out_a, lse_a = gpu.decode_inputs(sep)
    one = fresh()
    out_b, lse_b = gpu.decode_inputs(one, append=(c_new, k_new, pos))
    torch.cuda.synchronize()
    assert not torch.equal(sep.cache.view(torch.uint8), inp.cache.view(torch.uint8))
    assert torch.equal(sep.cache.view(torch.uint8), one.cache.view(torch.uint8))
    if sep.scales is not None:
        assert torch.equal(sep.scales, one.scales)
    assert torch.equal(out_a.view(torch.uint8), out_b.view(torch.uint8))
    assert torch.equal(lse_a, lse_b)
