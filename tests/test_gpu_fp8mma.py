"""The fp8 cache on the fp8 matrix cores (mla_decode_fp8mma_kernel: e4m3
codes as stored, query and weights as e4m3 hi + lo with power-of-two block
scales) against the oracle on the dequantised cache, at the fp8 tolerance;
and the same inputs through the widening kernel (MLA_FP8_KERNEL=widen),
which must agree with the oracle too."""

import os

import pytest
import torch

import synth
from test_gpu_decode import run_and_compare

pytestmark = pytest.mark.gpu


@pytest.fixture
def widen():
    os.environ["MLA_FP8_KERNEL"] = "widen"
    yield
    del os.environ["MLA_FP8_KERNEL"]


def test_fp8mma_tile_edges_contiguous(gpu):
    """Lengths around the 64-token tile: 1, 63, 64, 65, 127, 129, and a long
    ragged one, contiguous cache, the planned splits."""
    lengths = torch.tensor([1, 63, 64, 65, 127, 129, 3001], dtype=torch.int32)
    inp = synth.make_inputs(5, B=7, N=3001, lengths=lengths)
    run_and_compare(gpu, inp, "fp8")


@pytest.mark.parametrize("splits", [1, 2, 3, 16])
def test_fp8mma_forced_splits(gpu, splits):
    """Splits of whole 64-token tiles: one split of 2000 tokens (32 tiles,
    the last partial), and more, with the merge."""
    lengths = torch.tensor([2000, 777], dtype=torch.int32)
    inp = synth.make_inputs(5, B=2, N=2000, lengths=lengths)
    run_and_compare(gpu, inp, "fp8", num_splits=splits)


def test_fp8mma_paged_64_and_128_blocks(gpu):
    """Paged caches whose blocks hold whole tiles (64 and 128 tokens)."""
    lengths = torch.tensor([1000, 64, 1], dtype=torch.int32)
    for bs in (64, 128):
        inp = synth.make_inputs(5, B=3, N=1000, lengths=lengths, paged=True, block_size=bs)
        run_and_compare(gpu, inp, "fp8")


def test_fp8mma_against_widening_kernel(gpu, widen):
    """The widening kernel on the same inputs (and a paged cache with 32-token
    blocks, which always takes it) stays within tolerance as well."""
    lengths = torch.tensor([1000, 65], dtype=torch.int32)
    inp = synth.make_inputs(5, B=2, N=1000, lengths=lengths)
    run_and_compare(gpu, inp, "fp8")
    inp = synth.make_inputs(5, B=2, N=1000, lengths=lengths, paged=True, block_size=32)
    run_and_compare(gpu, inp, "fp8")
