"""Structure of the seeded synthetic workloads (CPU only)."""

import torch

import synth


def test_ragged_lengths_and_pool():
    lengths = synth.lengths_of(3, 64, 4096)
    assert lengths.dtype == torch.int32 and lengths.shape == (64,)
    assert int(lengths.min()) >= 1024 and int(lengths.max()) <= 4096
    assert torch.equal(lengths, synth.lengths_of(3, 64, 4096))   # seeded
    table, nblocks = synth.paged_layout(3, lengths)
    need = [(int(n) + 63) // 64 for n in lengths]
    assert nblocks == sum(need)
    used = torch.cat([table[b, :k] for b, k in enumerate(need)])
    assert torch.equal(torch.sort(used).values, torch.arange(nblocks, dtype=torch.int32))


def test_small_inputs_shapes_and_seeds():
    a = synth.make_inputs(2, B=2, N=100, H=32)
    b = synth.make_inputs(2, B=2, N=100, H=32)
    assert torch.equal(a.cache.view(torch.int16), b.cache.view(torch.int16))
    assert a.q_nope.shape == (2, 32, 128) and a.w_uk.shape == (32, 128, 512)
    assert a.w_uv.shape == (32, 512, 128) and a.cache.shape == (200, 576)
    assert a.cache.dtype == torch.bfloat16 and a.seq_capacity == 100
    std = a.w_uk.float().std().item()
    assert abs(std - 512 ** -0.5) < 0.01


def test_fp8_rows_span_code_range():
    x = synth.normal((50, 576), 1)
    codes, s = synth.fp8_rows(x)
    assert codes.dtype == torch.uint8 and s.dtype == torch.bfloat16
    deq = codes.view(torch.float8_e4m3fn).float() * s.float()[:, None]
    assert torch.allclose(deq, x, rtol=0.07, atol=0.02 * float(x.abs().max()))
    amax_code = codes.view(torch.float8_e4m3fn).float().abs().amax(1)
    assert float(amax_code.min()) >= 400
