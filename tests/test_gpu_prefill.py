"""Prefill / chunked prefill in the recompute mode (mla_prefill) against the
oracle's chunked_prefill, every (sequence, query, head) row: full prompts of
T = N tokens (one query tile, ragged tiles, several key tiles, the 4096-token
prompt the benchmark times), chunks after a context (contiguous and paged),
ragged lengths within a batch, and a sequence shorter than the chunk (its
first queries see no row: zeros and lse = -inf)."""

import math

import numpy as np
import pytest
import torch

import synth
from helpers import TOL, LSE_TOL, gathered_rows, gpu_f64, rel_err_rows, to_f64
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu


def run_case(gpu, B, T, lengths, paged, H=128, block_size=64, heads=None, seed=0):
    lengths = torch.tensor(lengths, dtype=torch.int32)
    N = int(lengths.max())
    print(f"[case] prefill B={B} T={T} lengths={lengths.tolist()} paged={paged} H={H} "
          f"block={block_size}", flush=True)
    inp = synth.make_inputs(2, B=B, N=N, H=H, lengths=lengths, paged=paged,
                            block_size=block_size)
    qn, qp = synth.prefill_queries(6100 + seed, B, T, H)
    dev = inp.to("cuda")
    lat, rope = gpu.split_cache(dev.cache)
    out, lse = gpu.prefill(qn.cuda(), qp.cuda(), dev.w_uk, dev.w_uv, lat, rope, dev.lengths,
                           N, seq_capacity=dev.seq_capacity, block_table=dev.block_table,
                           block_size=block_size)
    torch.cuda.synchronize()
    got = gpu_f64(out)
    got_lse = lse.cpu().double().numpy()
    assert np.isfinite(got).all()
    wuk, wuv = to_f64(inp.w_uk, "bf16"), to_f64(inp.w_uv, "bf16")
    qn64, qp64 = to_f64(qn, "bf16"), to_f64(qp, "bf16")
    hs = range(H) if heads is None else heads
    ref = np.zeros((B, T, H, 128))
    ref_lse = np.full((B, T, H), -math.inf)
    for b in range(B):
        C, R = gathered_rows(inp, b)
        for h in hs:
            ref[b, :, h], ref_lse[b, :, h] = orc.chunked_prefill(qn64[b, :, h], qp64[b, :, h],
                                                                 wuk[h], wuv[h], C, R, inp.scale)
    hs = list(hs)
    g, r = got[:, :, hs], ref[:, :, hs]
    gl, rl = got_lse[:, :, hs], ref_lse[:, :, hs]
    empty = np.isinf(rl)
    assert np.array_equal(np.isinf(gl), empty) and np.all(gl[empty] < 0)
    assert np.all(g[empty] == 0)
    err = rel_err_rows(g[~empty], r[~empty])
    lerr = float(np.max(np.abs(gl[~empty] - rl[~empty])))
    print(f"[result] normwise rel err {err:.3e} (tol {TOL['bf16']}), lse {lerr:.3e}, "
          f"{int(empty.sum())} empty rows", flush=True)
    assert err <= TOL["bf16"]
    assert lerr <= LSE_TOL["bf16"]


@pytest.mark.parametrize("T", [1, 31, 33, 1000])
def test_prefill_full_prompt(gpu, T):
    """T = N: every query of a prompt over the prompt itself (causal)."""
    run_case(gpu, 1, T, [T], paged=False, seed=T)


def test_prefill_4096_prompt(gpu):
    """The benchmark's prompt: B=1, T=N=4096, 128 heads."""
    run_case(gpu, 1, 4096, [4096], paged=False, seed=4096)


def test_prefill_chunk_after_context_paged(gpu):
    """Chunks of 300 queries after contexts of 1200, 400 and 0 tokens, paged
    cache with 32-token blocks."""
    run_case(gpu, 3, 300, [1500, 700, 300], paged=True, block_size=32, seed=7)


def test_prefill_ragged_contiguous(gpu):
    """Chunks of 64 queries over sequences of 1000, 65 and 64 rows."""
    run_case(gpu, 3, 64, [1000, 65, 64], paged=False, seed=8)


def test_prefill_sequence_shorter_than_chunk(gpu):
    """A chunk of 200 over a sequence of 150 rows: its first 50 queries see
    no row (zeros, lse -inf); the other sequence is a whole 200-token prompt."""
    run_case(gpu, 2, 200, [200, 150], paged=True, seed=9)


def test_prefill_32_heads(gpu):
    """32 heads (one (sequence, head) group per XCD slot), a prompt of 777."""
    run_case(gpu, 2, 777, [777, 777], paged=False, H=32, seed=10)


@pytest.mark.parametrize("order", ["0", "1"])
def test_prefill_work_orders(gpu, monkeypatch, order):
    """Both orders of the attention launch's workgroups (each (sequence,
    head) pair's query tiles in a row, or the longest tiles of all pairs
    first): chunks of 300 (three query tiles, the last ragged) after
    contexts of 1200, 400 and 0 tokens, 32 heads."""
    monkeypatch.setenv("MLA_PREFILL_ORDER", order)
    run_case(gpu, 3, 300, [1500, 700, 300], paged=False, H=32, seed=11)
