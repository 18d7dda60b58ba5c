"""The debug-checks build of the library (libmla_hip_debug.so, compiled with
MLA_DEBUG_CHECKS=1) against the release build.

The preconditions on device-resident integers (0 <= lengths[b] <= max_len,
block-table entries inside the cache, append positions inside a sequence's
capacity) cannot be checked by the host without a synchronisation. Both
builds clamp a violating value the same way (a length to [0, max_len], a
cache row outside the arrays to row 0, an append outside the capacity is
dropped), so no kernel reads or writes outside its buffers; the debug build
also sets the violation's bit in its error word (mla_debug_errors).

Checked here: on valid inputs the debug build returns the release build's
bits and an empty word; each kind of violation sets exactly its bit, and the
two builds still agree bit for bit. Every invalid value below is one of
those the kernels clamp."""

import dataclasses
import os

import pytest
import torch

import head_latent_attention_07_amd as mla
import synth

pytestmark = pytest.mark.gpu

LENGTHS = [300, 200, 1, 64]


@pytest.fixture(scope="module")
def dbg(gpu):
    path = os.path.join(os.path.dirname(mla.LIB_PATH), "libmla_hip_debug.so")
    if not os.path.exists(path):
        pytest.fail(f"debug-checks library not built: {path} (head_latent_attention_07_amd/build.py)")
    with mla.using(path):
        mla.debug_errors()          # start from a clear word
    return path


def on_both(dbg, fn):
    """fn() with the release build, then with the debug build (its error word
    read after the call). Returns (release result, debug result, word)."""
    rel = fn()
    torch.cuda.synchronize()
    with mla.using(dbg):
        got = fn()
        word = mla.debug_errors()
    return rel, got, word


def same_bits(a, b):
    return all(torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))
               for x, y in zip(a, b))


def small(cfg, **kw):
    return synth.make_inputs(cfg, B=4, N=300, lengths=torch.tensor(LENGTHS, dtype=torch.int32),
                             **kw)


CASES = [
    ("bf16 paged", dict(cfg=3, paged=True)),
    ("fp8 paged (fp8 matrix cores)", dict(cfg=5, paged=True)),
    ("fp8 contiguous", dict(cfg=2, cache_dtype="fp8")),
    ("f32 contiguous", dict(cfg=1)),
]


@pytest.mark.parametrize("name,spec", CASES, ids=[c[0] for c in CASES])
def test_valid_inputs_same_bits_no_errors(dbg, name, spec):
    spec = dict(spec)
    inp = small(spec.pop("cfg"), **spec).to("cuda")
    print(f"[case] debug build, valid inputs: {name}", flush=True)
    rel, got, word = on_both(dbg, lambda: mla.decode_inputs(inp))
    assert word == 0, hex(word)
    assert same_bits(rel, got)


def test_valid_decode_with_append(dbg):
    inp = small(3, paged=True).to("cuda")
    c_new, k_new = synth.append_inputs(900, inp.B, "bf16")
    pos = (inp.lengths - 1).contiguous()
    print("[case] debug build, decode with append, valid", flush=True)

    def run():
        x = dataclasses.replace(inp, cache=inp.cache.clone())
        return (*mla.decode_inputs(x, append=(c_new.cuda(), k_new.cuda(), pos)), x.cache)

    rel, got, word = on_both(dbg, run)
    assert word == 0, hex(word)
    assert same_bits(rel, got)


@pytest.mark.parametrize("name,spec", CASES, ids=[c[0] for c in CASES])
def test_length_out_of_range(dbg, name, spec):
    """lengths[0] > max_len (read as max_len) and lengths[1] < 0 (read as 0,
    an empty sequence: zeros and lse -inf)."""
    spec = dict(spec)
    inp = small(spec.pop("cfg"), **spec)
    bad = torch.tensor([inp.max_len + 50, -3] + LENGTHS[2:], dtype=torch.int32)
    inp = dataclasses.replace(inp, lengths=bad).to("cuda")
    print(f"[case] debug build, lengths {bad.tolist()} max_len {inp.max_len}: {name}", flush=True)
    rel, got, word = on_both(dbg, lambda: mla.decode_inputs(inp))
    assert word == mla.DEBUG_LENGTH, hex(word)
    assert same_bits(rel, got)
    out, lse = got
    assert not out[1].any() and bool(torch.isneginf(lse[1]).all())


@pytest.mark.parametrize("cfg", [3, 5], ids=["bf16", "fp8 matrix cores"])
def test_block_entry_out_of_range(dbg, cfg):
    """One entry past the block pool and one negative (both read cache row 0
    instead)."""
    inp = small(cfg, paged=True)
    table = inp.block_table.clone()
    num_blocks = inp.cache.shape[0] // inp.block_size
    table[0, 1] = num_blocks + 3
    table[1, 0] = -1
    inp = dataclasses.replace(inp, block_table=table).to("cuda")
    print(f"[case] debug build, block entries {num_blocks + 3} and -1 (pool {num_blocks}), "
          f"cfg {cfg}", flush=True)
    rel, got, word = on_both(dbg, lambda: mla.decode_inputs(inp))
    assert word == mla.DEBUG_BLOCK, hex(word)
    assert same_bits(rel, got)
    # the error word was cleared by the read: a valid call leaves it empty
    good = small(cfg, paged=True).to("cuda")
    _, _, word = on_both(dbg, lambda: mla.decode_inputs(good))
    assert word == 0, hex(word)


def test_append_position_out_of_range(dbg):
    """mla_cache_append with positions past the capacity and negative: those
    rows are not written (the others are), in both builds."""
    inp = small(3, paged=False, seq_capacity=320).to("cuda")
    cap = inp.seq_capacity
    pos = torch.tensor([cap + 5, -1, 10, cap - 1], dtype=torch.int32, device="cuda")
    c_new, k_new = [t.cuda() for t in synth.append_inputs(901, inp.B, "bf16")]
    print(f"[case] debug build, append positions {pos.tolist()} capacity {cap}", flush=True)

    def run():
        cache = inp.cache.clone()
        lat, rope = mla.split_cache(cache)
        mla.cache_append(c_new, k_new, pos, lat, rope, heads=inp.H, seq_capacity=cap)
        return (cache,)

    rel, got, word = on_both(dbg, run)
    assert word == mla.DEBUG_POSITION, hex(word)
    assert same_bits(rel, got)
    cache = got[0].view(inp.B, cap, -1)
    before = inp.cache.view(inp.B, cap, -1)
    assert torch.equal(cache[0], before[0]) and torch.equal(cache[1], before[1])
    assert not torch.equal(cache[2, 10], before[2, 10])
    assert not torch.equal(cache[3, cap - 1], before[3, cap - 1])


def test_prefill_block_entry_out_of_range(dbg):
    """A paged prefill (chunk of 100 queries) with one block entry past the
    pool: the debug build reports it, both builds read cache row 0 there."""
    lengths = torch.tensor([300, 200], dtype=torch.int32)
    inp = synth.make_inputs(2, B=2, N=300, lengths=lengths, paged=True)
    table = inp.block_table.clone()
    num_blocks = inp.cache.shape[0] // inp.block_size
    table[1, 2] = num_blocks + 9
    inp = dataclasses.replace(inp, block_table=table).to("cuda")
    qn, qp = [t.cuda() for t in synth.prefill_queries(6400, 2, 100, inp.H)]
    lat, rope = mla.split_cache(inp.cache)
    print(f"[case] debug build, prefill with block entry {num_blocks + 9} (pool {num_blocks})",
          flush=True)

    def run():
        return mla.prefill(qn, qp, inp.w_uk, inp.w_uv, lat, rope, inp.lengths, inp.max_len,
                           block_table=inp.block_table, block_size=inp.block_size)

    rel, got, word = on_both(dbg, run)
    assert word == mla.DEBUG_BLOCK, hex(word)
    assert same_bits(rel, got)


def test_length_aware_plan_length_out_of_range(dbg):
    """The length-aware plan reads the lengths in the absorb launch: a length
    past max_len and a negative one are reported there and clamped, as in
    the default plan."""
    inp = small(3, paged=True)
    bad = torch.tensor([inp.max_len + 7, -1] + LENGTHS[2:], dtype=torch.int32)
    inp = dataclasses.replace(inp, lengths=bad).to("cuda")
    print(f"[case] debug build, length-aware plan, lengths {bad.tolist()}", flush=True)
    rel, got, word = on_both(dbg, lambda: mla.decode_inputs(inp, length_aware=True))
    assert word == mla.DEBUG_LENGTH, hex(word)
    assert same_bits(rel, got)
