"""Pins of the oracle's number-format code against torch's independent
implementations of bfloat16 and float8_e4m3fn, and against values fixed by
the format definitions (CPU only)."""

import numpy as np
import torch

from oracle import mla_oracle as orc


def test_bf16_decode_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = orc.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all(both_nan | (mine == ref))


def test_e4m3_decode_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3fn_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all(both_nan | (mine == ref))
    # values fixed by the format definition
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6 and mine[0x38] == 1.0
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert np.sum(np.isnan(mine)) == 2


def test_e4m3_encode_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    vals = orc.e4m3fn_bits_to_f64(codes)
    assert np.array_equal(orc.e4m3fn_value_to_bits(vals), codes)


def test_bf16_encode_roundtrip():
    codes = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    vals = orc.bf16_bits_to_f64(codes)
    assert np.array_equal(orc.bf16_value_to_bits(vals), codes)


def test_round_to_bf16_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000) * 10.0 ** r.integers(-30, 30, 100000),
                        r.standard_normal(1000) * 1e-39]).astype(np.float32)
    mine = orc.round_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mine, ref)


def test_round_to_e4m3_matches_torch():
    r = np.random.default_rng(1)
    x = np.concatenate([r.uniform(-448, 448, 100000), r.uniform(-0.1, 0.1, 10000),
                        r.uniform(-2.0 ** -6, 2.0 ** -6, 10000)]).astype(np.float32)
    mine = orc.round_to_e4m3fn_sat(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(mine, ref)


def test_round_ties_to_even_and_saturation():
    # midpoints: 1 + 1/16 lies between 1 and 1.125 -> even mantissa (1);
    # 1 + 3/16 between 1.125 and 1.25 -> 1.25; 2^-10 between 0 and 2^-9 -> 0;
    # 3 * 2^-10 between 2^-9 and 2^-8 -> 2^-8 (mantissa 2 is even)
    x = np.array([1 + 1 / 16, 1 + 3 / 16, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, 1e6, -1e6])
    assert list(orc.round_to_e4m3fn_sat(x)) == [1.0, 1.25, 0.0, 2.0 ** -8, 448.0, 448.0, -448.0]
    # bf16: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1
    assert orc.round_to_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]))[0] == 1.0
    assert orc.round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_fp8_row_scale_rules():
    # all-zero row -> 1; amax 448 -> 1 exactly; amax 896 -> 2
    assert orc.fp8_row_scale(np.zeros(576, np.float32)) == 1.0
    row = np.zeros(576, np.float32)
    row[3] = -448.0
    assert orc.fp8_row_scale(row) == 1.0
    row[7] = 896.0
    assert orc.fp8_row_scale(row) == 2.0
    row = np.zeros(576, np.float32)
    row[0] = 1e-40
    assert orc.fp8_row_scale(row) == 2.0 ** -126


def test_append_row_fp8_codes():
    """A row with one value at +896 and one at -1: scale 2, codes 0x7E (448)
    and the code of -0.5 (0xB0: sign 1, exponent 6, mantissa 0)."""
    c = np.zeros(512)
    c[0] = 896.0
    c[1] = -1.0
    lat, rope, scale, codes = orc.append_row(c, np.zeros(64), 0, "fp8")
    assert scale == 2.0
    assert codes[0] == 0x7E and codes[1] == 0xB0 and codes[2] == 0
    assert lat[0] == 896.0 and lat[1] == -1.0


def test_append_row_bf16_copies_latent_exactly():
    r = np.random.default_rng(3)
    c = orc.round_to_bf16(r.standard_normal(512))
    lat, rope, scale, codes = orc.append_row(c, r.standard_normal(64), 5, "bf16")
    assert np.array_equal(lat, c) and scale is None
