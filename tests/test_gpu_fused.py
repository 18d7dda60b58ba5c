"""Offline absorption (mla_fuse_weights + mla_decode_fused) against the
oracle: the fused weights against the oracle's own fusion, and the decode
from model-width input to model-width output against the unfused
definition (decode_model_io: q_nope = W_Q x per head, attention over the
decompressed keys and values, y = sum_h o_h W_O[h])."""

import numpy as np
import pytest
import torch

import synth
from helpers import LSE_TOL, TOL, gathered_rows, gpu_f64, rel_err_rows, to_f64
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu


def test_fuse_weights_against_oracle(gpu):
    """W_QK[h] = W_UK[h]^T W_Q[h] and W_VO = W_UV[h] W_O[h] (stored
    [d_model, 512 H]), every row of both, 32 heads, d_model 320."""
    H, D = 32, 320
    inp = synth.make_inputs(2, B=1, N=8, H=H)
    _, w_q, w_o = synth.model_io_inputs(4200, 1, H, D)
    print(f"[case] fuse weights H={H} d_model={D}", flush=True)
    w_qk, w_vo = gpu.fuse_weights(w_q.cuda(), inp.w_uk.cuda(), inp.w_uv.cuda(), w_o.cuda())
    torch.cuda.synchronize()
    wq, wuk, wuv, wo = (to_f64(t, "bf16") for t in (w_q, inp.w_uk, inp.w_uv, w_o))
    ref_qk = np.stack([orc.fuse_query_weight(wq[h], wuk[h]) for h in range(H)])   # [H, 512, D]
    ref_vo = np.stack([orc.fuse_output_weight(wuv[h], wo[h]) for h in range(H)])  # [H, 512, D]
    got_qk = gpu_f64(w_qk)
    got_vo = gpu_f64(w_vo).reshape(D, H, 512).transpose(1, 2, 0)                  # -> [H, 512, D]
    e1 = rel_err_rows(got_qk, ref_qk)
    e2 = rel_err_rows(got_vo, ref_vo)
    print(f"[result] W_QK rows {e1:.3e}, W_VO rows {e2:.3e} (one bf16 rounding: <= 2^-8)",
          flush=True)
    assert e1 <= 2.0 ** -8 and e2 <= 2.0 ** -8


def run_fused(gpu, B, N, H, D, lengths, paged, cache_dtype="bf16", seed=0, sample=None):
    lengths = torch.tensor(lengths, dtype=torch.int32)
    print(f"[case] decode_fused B={B} N={N} H={H} d_model={D} paged={paged} cache={cache_dtype}",
          flush=True)
    inp = synth.make_inputs(3, B=B, N=N, H=H, lengths=lengths, paged=paged,
                            cache_dtype=cache_dtype)
    x, w_q, w_o = synth.model_io_inputs(4300 + seed, B, H, D)
    dev = inp.to("cuda")
    w_qk, w_vo = gpu.fuse_weights(w_q.cuda(), dev.w_uk, dev.w_uv, w_o.cuda())
    lat, rope = gpu.split_cache(dev.cache)
    out, lse = gpu.decode_fused(x.cuda(), dev.q_pe, w_qk, w_vo, lat, rope, dev.lengths,
                                dev.max_len, seq_capacity=dev.seq_capacity,
                                block_table=dev.block_table, block_size=dev.block_size,
                                scales=dev.scales)
    torch.cuda.synchronize()
    got, got_lse = gpu_f64(out), lse.cpu().double().numpy()
    del w_qk, w_vo
    bs = range(B) if sample is None else sample
    xq, wq, wo = to_f64(x, "bf16"), to_f64(w_q, "bf16"), to_f64(w_o, "bf16")
    wuk, wuv, qp = to_f64(inp.w_uk, "bf16"), to_f64(inp.w_uv, "bf16"), to_f64(inp.q_pe, "bf16")
    ref = np.empty((len(bs), D))
    ref_lse = np.empty((len(bs), H))
    for i, b in enumerate(bs):
        C, R = gathered_rows(inp, b)
        ref[i], ref_lse[i] = orc.decode_model_io(xq[b], qp[b], wq, wuk, wuv, wo, C, R, inp.scale)
    bs = list(bs)
    err = rel_err_rows(got[bs], ref)
    lerr = float(np.max(np.abs(got_lse[bs] - ref_lse)))
    tol = TOL[cache_dtype]
    print(f"[result] y normwise rel err {err:.3e} (tol {tol}), lse {lerr:.3e} over "
          f"{len(bs)} sequences", flush=True)
    assert err <= tol
    assert lerr <= LSE_TOL[cache_dtype]


def test_decode_fused_small_paged(gpu):
    run_fused(gpu, 3, 1000, 32, 512, [300, 1, 1000], paged=True, seed=1)


def test_decode_fused_small_fp8_contiguous(gpu):
    run_fused(gpu, 2, 777, 64, 256, [777, 64], paged=False, cache_dtype="fp8", seed=2)


def test_decode_fused_full_size(gpu):
    """The benchmark's shapes: B=64, H=128, N=4096 paged bf16, d_model 7168;
    four sequences compared (every output of each)."""
    run_fused(gpu, 64, 4096, 128, 7168, [4096] * 64, paged=True, seed=3, sample=[0, 21, 42, 63])
