"""The length-aware split plan (mla_decode_options.length_aware, bf16 cache):
the device cuts each sequence by its own length (up to twice the default
split count for the longest), the attention launch walks the resulting work
items, and the merge reads each sequence's own number of partials. The result
is the same softmax as with the default plan; every case is compared with
the oracle, and the full-size ragged workload on every (sequence, head)."""

import numpy as np
import pytest
import torch

import synth
from helpers import LSE_TOL, TOL, gpu_f64, oracle_decode, oracle_decode_seq, rel_err_rows

pytestmark = pytest.mark.gpu


def check(mla, inp, batch_ids=None, heads=None, **kw):
    dev = inp.to("cuda")
    print(f"[case] length-aware B={inp.B} H={inp.H} max_len={inp.max_len} paged={inp.paged} "
          f"lengths[:8]={inp.lengths[:8].tolist()} kw={sorted(kw)}", flush=True)
    out, lse = mla.decode_inputs(dev, length_aware=True, **kw)
    base, base_lse = mla.decode_inputs(dev, **kw)
    torch.cuda.synchronize()
    g, gl = gpu_f64(out), lse.cpu().double().numpy()
    assert np.isfinite(g).all()
    ref, ref_lse = oracle_decode(inp, batch_ids=batch_ids, heads=heads)
    bs = list(range(inp.B)) if batch_ids is None else list(batch_ids)
    hs = list(range(inp.H)) if heads is None else list(heads)
    g, gl = g[bs][:, hs], gl[bs][:, hs]
    ref, ref_lse = ref[:, hs], ref_lse[:, hs]
    err = rel_err_rows(g, ref)
    fin = np.isfinite(ref_lse)
    assert (np.isneginf(gl) == ~fin).all()
    lerr = float(np.max(np.abs(gl[fin] - ref_lse[fin]))) if fin.any() else 0.0
    # the default plan on the same inputs (other split points: other rounding)
    berr = rel_err_rows(gpu_f64(out), gpu_f64(base))
    print(f"[result] rel err {err:.3e} (tol {TOL['bf16']}), lse {lerr:.3e}; "
          f"vs default plan {berr:.3e}", flush=True)
    assert err <= TOL["bf16"], err
    assert lerr <= LSE_TOL["bf16"], lerr
    assert berr <= TOL["bf16"], berr


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contiguous"])
def test_edge_lengths(gpu, paged):
    """Empty, single-row, tile-edge and longest sequences together (B=8):
    the longest gets more splits than the default plan gives it."""
    lengths = torch.tensor([0, 1, 31, 32, 33, 700, 2500, 3001], dtype=torch.int32)
    inp = synth.make_inputs(3, B=8, N=3001, lengths=lengths, paged=paged)
    check(gpu, inp)


def test_one_long_many_short(gpu):
    """One 4096-token sequence and 63 short ones: the split length is held at
    max_len / (2 x default splits), the long sequence takes 8 work items."""
    lengths = torch.tensor([4096] + [1 + 7 * i for i in range(63)], dtype=torch.int32)
    inp = synth.make_inputs(3, B=64, N=4096, lengths=lengths, paged=True)
    check(gpu, inp, batch_ids=[0, 1, 17, 63], heads=list(range(0, 128, 9)))


def test_many_sequences(gpu):
    """B=130 (five chunks of 32 in the merge, the last ragged), lengths
    U[1, 2000]."""
    g = torch.Generator().manual_seed(4242)
    lengths = torch.randint(1, 2001, (130,), generator=g, dtype=torch.int64).to(torch.int32)
    inp = synth.make_inputs(3, B=130, N=2000, lengths=lengths, paged=True)
    check(gpu, inp, batch_ids=[0, 31, 32, 64, 127, 129], heads=list(range(0, 128, 11)))


def test_with_append(gpu):
    """The decode call appends the new rows (absorb launch), then plans on
    the lengths that include them."""
    from oracle import mla_oracle as orc
    from helpers import to_f64
    lengths = torch.tensor([5, 900, 64, 2048, 1], dtype=torch.int32)
    inp = synth.make_inputs(3, B=5, N=2048, lengths=lengths, paged=True)
    c_new, k_new = synth.append_inputs(7100, inp.B, "bf16")
    pos = inp.lengths - 1
    dev = inp.to("cuda")
    out, lse = gpu.decode_inputs(dev, length_aware=True,
                                 append=(c_new.cuda(), k_new.cuda(), pos.cuda()))
    torch.cuda.synchronize()
    ref_inp = synth.make_inputs(3, B=5, N=2048, lengths=lengths, paged=True)
    table = inp.block_table.numpy()
    for b in range(inp.B):
        p = int(pos[b])
        lat, rope, _, _ = orc.append_row(to_f64(c_new[b], "bf16"), to_f64(k_new[b], "bf16"), p,
                                         "bf16")
        row = orc.paged_row(table, b, p, inp.block_size)
        ref_inp.cache[row] = torch.from_numpy(
            np.concatenate([lat, rope]).astype(np.float32)).to(torch.bfloat16)
    ref, ref_lse = oracle_decode(ref_inp)
    err = rel_err_rows(gpu_f64(out), ref)
    lerr = float(np.max(np.abs(lse.cpu().double().numpy() - ref_lse)))
    print(f"[result] length-aware with append: rel err {err:.3e}, lse {lerr:.3e}", flush=True)
    assert err <= TOL["bf16"] and lerr <= LSE_TOL["bf16"]


def test_config3_full_every_row(gpu):
    """The ragged benchmark workload (B=64, lengths U[1024, 4096], paged):
    every (sequence, head) row against the all-heads absorbed oracle."""
    inp = synth.make_inputs(3)
    print(f"[case] length-aware config 3 full, sum of lengths {int(inp.lengths.sum())}",
          flush=True)
    out, lse = gpu.decode_inputs(inp.to("cuda"), length_aware=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode_seq(inp)
    err = rel_err_rows(gpu_f64(out), ref)
    lerr = float(np.max(np.abs(lse.cpu().double().numpy() - ref_lse)))
    print(f"[result] config 3 length-aware all rows: rel err {err:.3e}, lse {lerr:.3e}",
          flush=True)
    assert err <= TOL["bf16"] and lerr <= LSE_TOL["bf16"]


@pytest.mark.parametrize("H", [32, 64, 256])
def test_head_counts(gpu, H):
    """One wave (H=32), two waves (H=64) per workgroup, and two head groups
    per sequence (H=256): the work items are shared by the head groups."""
    lengths = torch.tensor([1500, 40, 700, 1], dtype=torch.int32)
    inp = synth.make_inputs(3, B=4, N=1500, H=H, lengths=lengths, paged=True)
    check(gpu, inp, heads=list(range(0, H, 7)))



def _plan_layout(B, H, max_len, cus):
    """Offsets of the length-aware plan in the decode workspace (bf16 path):
    the default plan's splits S (as the library makes it for this CU count),
    2S partial slots, B*S work items, then the splits per sequence."""
    cdiv = lambda a, b: -(-a // b)
    al = lambda x: (x + 255) // 256 * 256
    S = min(cdiv(cus, B), cdiv(max_len, 64))
    S = max(1, min(S, cdiv(max_len, 32)))
    S = max(S, cdiv(max_len, 64 * 32))
    ts = cdiv(cdiv(max_len, S), 32) * 32
    S = cdiv(max_len, ts)
    slots, nitems = 2 * S, B * S
    rows = B * slots * H
    po = al(B * H * 576 * 2)
    ps = al(po + rows * 512 * 2)
    pl = al(ps + rows * 4)
    items = al(pl + rows * 4)
    nsplit = al(items + nitems * 16)
    return S, ts, slots, nitems, items, nsplit


def test_plan_is_the_smallest_fitting_split(gpu):
    """The plan the device made, read back from the workspace: every
    sequence cut into n_b = max(1, ceil(len_b / c)) consecutive items
    covering [0, len_b) in order, the unused items marked empty, and c the
    smallest multiple of 32 tokens in [max_len / slots, default split
    length] for which the splits of all sequences fit in the work items."""
    g = torch.Generator().manual_seed(77)
    lengths = torch.randint(1, 4097, (48,), generator=g, dtype=torch.int64).to(torch.int32)
    lengths[5] = 0
    lengths[9] = 4096
    inp = synth.make_inputs(3, B=48, N=4096, lengths=lengths, paged=True).to("cuda")
    B, H = inp.B, inp.H
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S, ts, slots, nitems, items_off, nsplit_off = _plan_layout(B, H, inp.max_len, cus)
    act = gpu.dtype_code(inp.q_nope.dtype)
    wsz = gpu.workspace_size(H, B, inp.max_len, act, act, 0, True)
    assert wsz == (nsplit_off + B * 4 + 255) // 256 * 256
    ws = torch.zeros(wsz, dtype=torch.uint8, device="cuda")
    print(f"[case] plan readback B={B} S={S} slots={slots} items={nitems}", flush=True)
    gpu.decode_inputs(inp, workspace=ws, length_aware=True)
    torch.cuda.synchronize()
    w = ws.cpu()
    items = w[items_off:items_off + nitems * 16].view(torch.int32).view(nitems, 4).tolist()
    nsplit = w[nsplit_off:nsplit_off + B * 4].view(torch.int32).tolist()
    lens = [max(0, min(int(x), inp.max_len)) for x in lengths]
    cdiv = lambda a, b: -(-a // b)
    # the split length: the first item of a sequence with two or more
    c = next(t1 - t0 for b_, s_, t0, t1 in items if b_ >= 0 and s_ == 0 and nsplit[b_] > 1)
    assert c % 32 == 0 and cdiv(inp.max_len, slots) <= c <= ts, (c, ts)
    count = lambda cc: sum(max(1, cdiv(n, cc)) for n in lens)
    assert count(c) <= nitems
    if c - 32 >= max(32, cdiv(cdiv(inp.max_len, slots), 32) * 32):
        assert count(c - 32) > nitems
    q = 0
    for b in range(B):
        n = max(1, cdiv(lens[b], c))
        assert nsplit[b] == n
        for s in range(n):
            assert items[q] == [b, s, s * c, min((s + 1) * c, lens[b])], (q, items[q])
            q += 1
    assert q == sum(nsplit) <= nitems
    assert all(it[0] == -1 for it in items[q:])
    print(f"[result] c={c} tokens, {q} of {nitems} items used", flush=True)
