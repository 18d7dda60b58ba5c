"""Parity at the full workload sizes, in the launch configuration the
benchmark times: sampled sequences and heads are compared with the oracle
one by one (the oracle cannot afford every output at these sizes)."""

import numpy as np
import pytest
import torch

import synth
from helpers import LSE_TOL, TOL, gpu_f64, oracle_decode, rel_err_rows

pytestmark = pytest.mark.gpu


def check_sampled(gpu, inp, batch_ids, heads, tol_key, **kw):
    print(f"[case] cfg={inp.cfg} B={inp.B} max_len={inp.max_len} paged={inp.paged} "
          f"sample b={batch_ids} heads={len(heads)}", flush=True)
    out, lse = gpu.decode_inputs(inp.to("cuda"), **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ref, ref_lse = oracle_decode(inp, batch_ids=batch_ids, heads=heads)
    g = gpu_f64(out)[batch_ids][:, heads]
    err = rel_err_rows(g, ref[:, heads])
    lerr = float(np.max(np.abs(lse.cpu().double().numpy()[batch_ids][:, heads] - ref_lse[:, heads])))
    print(f"[result] sampled normwise rel err {err:.3e} (tol {TOL[tol_key]}), lse {lerr:.3e}",
          flush=True)
    assert err <= TOL[tol_key]
    assert lerr <= LSE_TOL[tol_key]
    return out, lse


HEADS = list(range(0, 128, 5))


def test_config3_ragged_paged(gpu):
    """B=64, lengths U[1024, 4096], paged 64-token blocks."""
    inp = synth.make_inputs(3)
    b = [0, 17, int(torch.argmax(inp.lengths)), int(torch.argmin(inp.lengths))]
    check_sampled(gpu, inp, b, HEADS, "bf16")


def test_config3_uniform_paged(gpu):
    """B=64, every N=4096, paged: the benchmark workload."""
    inp = synth.make_inputs("3u")
    check_sampled(gpu, inp, [0, 63], HEADS, "bf16")


def test_config3_uniform_paged_step_with_append(gpu):
    """The benchmark step itself: B=64, N=4096, paged, one decode call that
    first appends each sequence's new token (position N-1, RoPE on its key)
    in the absorb launch. The oracle makes the appended rows with its own
    append and decodes the resulting cache."""
    from oracle import mla_oracle as orc
    from helpers import to_f64
    inp = synth.make_inputs("3u")
    c_new, k_new = synth.append_inputs(7000, inp.B, "bf16")
    pos = inp.lengths - 1
    dev = inp.to("cuda")
    print("[case] 3u step with append", flush=True)
    out, lse = gpu.decode_inputs(dev, append=(c_new.cuda(), k_new.cuda(), pos.cuda()))
    torch.cuda.synchronize()
    batch_ids = [0, 31, 63]
    table = inp.block_table.numpy()
    for b in batch_ids:
        p = int(pos[b])
        lat, rope, _, _ = orc.append_row(to_f64(c_new[b], "bf16"), to_f64(k_new[b], "bf16"), p, "bf16")
        row = orc.paged_row(table, b, p, inp.block_size)
        inp.cache[row] = torch.from_numpy(np.concatenate([lat, rope]).astype(np.float32)).to(torch.bfloat16)
    ref, ref_lse = oracle_decode(inp, batch_ids=batch_ids, heads=HEADS)
    g = gpu_f64(out)[batch_ids][:, HEADS]
    err = rel_err_rows(g, ref[:, HEADS])
    lerr = float(np.max(np.abs(lse.cpu().double().numpy()[batch_ids][:, HEADS] - ref_lse[:, HEADS])))
    print(f"[result] sampled normwise rel err {err:.3e}, lse {lerr:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert lerr <= LSE_TOL["bf16"]


def test_config4_long_context(gpu):
    """B=4, N=131072 (128K context), contiguous: many splits per sequence."""
    inp = synth.make_inputs(4)
    check_sampled(gpu, inp, [1], list(range(0, 128, 16)), "bf16")


def test_config5_fp8_layer_sample(gpu):
    """fp8 cache, B=32, N=32768: two of the 61 layers (each layer has its own
    seeded weights, queries and cache), sampled sequences and heads."""
    for layer in (0, 60):
        inp = synth.make_inputs(5, layer=layer, gen_device="cuda")
        check_sampled(gpu, inp.to("cpu"), [3], list(range(0, 128, 32)), "fp8")
        del inp
        torch.cuda.empty_cache()
