"""GPU parity of the HIP decode path against the CPU oracle (element-wise on
the same seeded inputs), through the C ABI."""

import numpy as np
import pytest
import torch

import synth
from helpers import LSE_TOL, TOL, gpu_f64, oracle_decode, rel_err_rows

pytestmark = pytest.mark.gpu


def run_and_compare(mla, inp, tol_key, batch_ids=None, heads=None, lse_rel=False, **kw):
    dev = inp.to("cuda")
    print(f"[case] cfg={inp.cfg} B={inp.B} H={inp.H} max_len={inp.max_len} "
          f"cache={inp.cache_dtype} paged={inp.paged} kw={kw}", flush=True)
    out, lse = mla.decode_inputs(dev, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(inp, batch_ids=batch_ids, heads=heads)
    g = gpu_f64(out)
    gl = lse.cpu().double().numpy()
    if batch_ids is not None:
        g, gl = g[batch_ids], gl[batch_ids]
    if heads is not None:
        g, gl = g[:, heads], gl[:, heads]
        ref, ref_lse = ref[:, heads], ref_lse[:, heads]
    err = rel_err_rows(g, ref)
    den = np.maximum(np.abs(ref_lse), 1.0) if lse_rel else 1.0
    lerr = float(np.nanmax(np.abs(gl - ref_lse) / den)) if np.isfinite(ref_lse).any() else 0.0
    print(f"[result] max normwise rel err {err:.3e} (tol {TOL[tol_key]}), lse abs err {lerr:.3e}",
          flush=True)
    assert err <= TOL[tol_key], err
    assert lerr <= LSE_TOL[tol_key], lerr
    return out, lse


def test_config1_fp32_full(gpu):
    """fp32, B=1, H=16, N=512: every output against the oracle at 1e-4."""
    run_and_compare(gpu, synth.make_inputs(1), "f32")


def test_fp32_ragged_splits(gpu):
    """fp32 path: ragged lengths, several splits, a tail not a multiple of 32."""
    lengths = torch.tensor([1, 33, 700, 1500], dtype=torch.int32)
    inp = synth.make_inputs(1, B=4, N=1500, H=16, lengths=lengths)
    run_and_compare(gpu, inp, "f32")
    run_and_compare(gpu, inp, "f32", num_splits=5)


@pytest.mark.parametrize("H", [32, 64, 128])
def test_bf16_ragged_contiguous(gpu, H):
    """bf16 MFMA path for each wave count (H/32 = 1, 2, 4 waves per workgroup):
    lengths 1 (single row), 31 (partial first tile), 33 (tile + 1 row),
    320 and 1001 (several tiles and a ragged tail)."""
    lengths = torch.tensor([1, 31, 33, 320, 1001], dtype=torch.int32)
    inp = synth.make_inputs(2, B=5, N=1001, H=H, lengths=lengths)
    run_and_compare(gpu, inp, "bf16")


def test_bf16_paged_small(gpu):
    lengths = torch.tensor([64, 65, 130, 1000], dtype=torch.int32)
    inp = synth.make_inputs(3, B=4, N=1000, lengths=lengths, paged=True)
    run_and_compare(gpu, inp, "bf16")


@pytest.mark.parametrize("splits", [1, 2, 5, 7, 8, 32])
def test_split_invariance(gpu, splits):
    """The split-KV merge is an exact re-association of the softmax: every
    forced split count agrees with the oracle."""
    lengths = torch.tensor([1024, 700], dtype=torch.int32)
    inp = synth.make_inputs(2, B=2, N=1024, lengths=lengths)
    run_and_compare(gpu, inp, "bf16", num_splits=splits)


@pytest.mark.parametrize("N,splits", [(2240, 70), (4096, 128)])
def test_many_splits(gpu, N, splits):
    """More than 64 splits: the merge takes its weights 64 splits at a time
    (70 = one chunk of 64 and a chunk of 6 with a partial group of 4)."""
    lengths = torch.tensor([N, N - 700, 33], dtype=torch.int32)
    inp = synth.make_inputs(2, B=3, N=N, lengths=lengths)
    run_and_compare(gpu, inp, "bf16", num_splits=splits)


@pytest.mark.parametrize("groups", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("N,splits", [(1024, 7), (2240, 70)])
def test_merge_levels(gpu, monkeypatch, N, splits, groups):
    """Rows of more than 4 splits, merged in one pass (groups=0: the merge
    with the weight table) or first folded into 1-4 groups of consecutive
    splits that the second pass merges: 7 splits as 7, 4+3, 3+3+1, 2+2+2+1;
    70 as 70 (16 splits per step, five steps, the last of 6), 35+35,
    24+24+22, 18+18+18+16. The sequence of 33 tokens makes whole groups of
    empty splits."""
    monkeypatch.setenv("MLA_MERGE_GROUPS", str(groups))
    lengths = torch.tensor([N, N - 700, 33], dtype=torch.int32)
    inp = synth.make_inputs(2, B=3, N=N, lengths=lengths)
    run_and_compare(gpu, inp, "bf16", num_splits=splits)


@pytest.mark.parametrize("merge8", ["1", "0"])
@pytest.mark.parametrize("splits", [5, 8])
def test_merge_eight_slots(gpu, monkeypatch, merge8, splits):
    """5-8 partials per row: the row merge with 8 slots in one launch
    (MLA_MERGE8=1, the default) or the general paths (0), for 40 sequences
    (a full chunk of 32 and a chunk of 8) including short ones whose later
    splits are empty."""
    monkeypatch.setenv("MLA_MERGE8", merge8)
    lengths = torch.tensor([(97 * i) % 700 + 1 for i in range(39)] + [700], dtype=torch.int32)
    inp = synth.make_inputs(2, B=40, N=700, lengths=lengths)
    run_and_compare(gpu, inp, "bf16", batch_ids=[0, 5, 31, 32, 38, 39], num_splits=splits)


@pytest.mark.parametrize("cols", [1, 2])
@pytest.mark.parametrize("splits", [3, 22])
def test_merge_column_split(gpu, monkeypatch, cols, splits):
    """The merge of at most 4 partials with all 128 output columns per
    workgroup (cols=1) or 64 (cols=2: two workgroups per head and chunk of
    32 sequences): 40 sequences (a full chunk and a chunk of 8), 3 splits
    merged directly, 22 folded into two groups first. The oracle checks
    sequences from both chunks, the short ones included."""
    monkeypatch.setenv("MLA_COMBINE_COLS", str(cols))
    lengths = torch.tensor([(97 * i) % 700 + 1 for i in range(39)] + [700], dtype=torch.int32)
    inp = synth.make_inputs(2, B=40, N=700, lengths=lengths)
    run_and_compare(gpu, inp, "bf16", batch_ids=[0, 5, 31, 32, 38, 39], num_splits=splits)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 0])
def test_late_large_score_restart(gpu, cache_dtype, splits):
    """Rows deep into the split (tokens 600, 610, 620, 630) are each set along
    the part of one head's absorbed query (heads 3, 40, 77, 120: one per
    wave) that is orthogonal to every other head's, scaled so that for that
    head they outscore the first tile, the split's fixed exponent reference,
    by far more than 64 in log2 units, while the other heads barely see them:
    the weights overflow and the split is recomputed against its true
    maximum. splits=0: the planned split count."""
    from helpers import gathered_rows, to_f64
    lengths = torch.tensor([700, 300], dtype=torch.int32)
    inp = synth.make_inputs(2 if cache_dtype == "bf16" else 5, B=2, N=700, lengths=lengths,
                            cache_dtype=cache_dtype)
    qlat = np.einsum("hn,hnc->hc", to_f64(inp.q_nope[0], "bf16"), to_f64(inp.w_uk, "bf16"))
    heads, rows = [3, 40, 77, 120], [600, 610, 620, 630]
    for hh, row in zip(heads, rows):
        others = np.delete(qlat, hh, axis=0)
        coef = np.linalg.lstsq(others.T, qlat[hh], rcond=None)[0]
        qperp = qlat[hh] - others.T @ coef
        x = torch.zeros((1, 576), dtype=torch.float32)
        x[0, :512] = torch.from_numpy(100.0 / (qperp @ qperp * inp.scale * np.log2(np.e)) * qperp)
        if cache_dtype == "bf16":
            inp.cache[row] = x[0].to(torch.bfloat16)
        else:
            codes, scale = synth.fp8_rows(x)
            inp.cache[row], inp.scales[row] = codes[0], scale[0]
    c, r = gathered_rows(inp, 0)
    sc = (c @ qlat.T + r @ to_f64(inp.q_pe[0], "bf16").T) * inp.scale * np.log2(np.e)
    assert (sc[rows, heads] - sc[:32, heads].max(axis=0) > 64).all()   # the premise
    assert np.abs(np.delete(sc[rows], heads, axis=1)).max() < 4       # and only for them
    # lse gated relative to its size: the target heads' lse is ~70, and the
    # bf16 rounding of the absorbed query moves a dominating score, and so
    # the lse, by up to 2^-9 of itself
    run_and_compare(gpu, inp, "bf16" if cache_dtype == "bf16" else "fp8", num_splits=splits,
                    lse_rel=True)


def test_paged_equals_contiguous_bitwise(gpu):
    """Block-table indexing is exact: the same rows, placed in a permuted
    pool of 64-token blocks, give bit-identical outputs under the same split
    plan."""
    lengths = torch.tensor([1000, 257, 64], dtype=torch.int32)
    inp = synth.make_inputs(2, B=3, N=1024, lengths=lengths, seq_capacity=1024)
    bs = 64
    nb = 1024 // bs
    perm = torch.randperm(3 * nb, generator=torch.Generator().manual_seed(5))
    table = perm.view(3, nb).to(torch.int32)
    pool = torch.empty_like(inp.cache)
    for b in range(3):
        for j in range(nb):
            pool[int(table[b, j]) * bs:(int(table[b, j]) + 1) * bs] = \
                inp.cache[b * 1024 + j * bs:b * 1024 + (j + 1) * bs]
    paged = synth.DecodeInputs(**{**inp.__dict__, "cache": pool, "block_table": table,
                                  "seq_capacity": 0, "block_size": bs})
    o1, l1 = gpu.decode_inputs(inp.to("cuda"), num_splits=3)
    o2, l2 = gpu.decode_inputs(paged.to("cuda"), num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_empty_sequence(gpu):
    """len 0: output 0 and lse = -inf; the other sequence is unaffected."""
    lengths = torch.tensor([0, 40], dtype=torch.int32)
    inp = synth.make_inputs(2, B=2, N=64, lengths=lengths)
    out, lse = gpu.decode_inputs(inp.to("cuda"))
    torch.cuda.synchronize()
    assert torch.all(out[0].float() == 0)
    assert torch.all(torch.isneginf(lse[0]))
    run_and_compare(gpu, inp, "bf16", batch_ids=[1])


def test_fp8_cache_small(gpu):
    """fp8 e4m3 cache with a bf16 scale per row, compared on the dequantised
    cache at 3e-2."""
    lengths = torch.tensor([1, 100, 777], dtype=torch.int32)
    inp = synth.make_inputs(5, B=3, N=777, lengths=lengths)
    run_and_compare(gpu, inp, "fp8")
    run_and_compare(gpu, inp, "fp8", num_splits=4)


@pytest.mark.parametrize("H", [32, 64])
def test_fp8_cache_fewer_waves(gpu, H):
    """fp8 cache with H/32 = 1 or 2 waves per workgroup (with one wave a
    lane's staged pieces outnumber the first step's MFMA slots): lengths 1,
    33, 300 and 777 (several tiles, a ragged tail)."""
    lengths = torch.tensor([1, 33, 300, 777], dtype=torch.int32)
    inp = synth.make_inputs(5, B=4, N=777, H=H, lengths=lengths)
    run_and_compare(gpu, inp, "fp8")
    run_and_compare(gpu, inp, "fp8", num_splits=3)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_size", [32, 128])
def test_paged_block_sizes(gpu, cache_dtype, block_size):
    """Paged caches with 32- and 128-token blocks (any multiple of the
    32-token tile): 32 puts every tile in its own block, 128 four per block."""
    lengths = torch.tensor([1000, 129, 32, 500], dtype=torch.int32)
    inp = synth.make_inputs(3, B=4, N=1000, lengths=lengths, paged=True, block_size=block_size,
                            cache_dtype=cache_dtype)
    run_and_compare(gpu, inp, cache_dtype)


def test_config2_full(gpu):
    """bf16, B=1, H=128, N=4096 (DeepSeek-V3 shape): every output."""
    run_and_compare(gpu, synth.make_inputs(2), "bf16")
