"""The C-ABI library: it loads, exports every symbol include/mla.h declares,
and rejects invalid arguments before launching anything (CPU only: no call
here reaches a kernel)."""

import ctypes
import os
import re

import pytest

import head_latent_attention_07_amd as mla

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mla.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(mla.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(5):
        assert mla.status_string(code).startswith("MLA_")
    assert mla.status_string(99) == "MLA_ERR_UNKNOWN"


def test_cache_bytes_per_token():
    # 576 numbers per token per layer; fp8 adds a 2-byte scale
    assert mla.cache_bytes_per_token(mla.MLA_BF16) == 1152
    assert mla.cache_bytes_per_token(mla.MLA_F32) == 2304
    assert mla.cache_bytes_per_token(mla.MLA_FP8_E4M3) == 578
    assert mla.cache_bytes_per_token(7) == 0
    assert mla.cache_bytes_per_token(mla.MLA_BF16, 0, 64) == 0


def test_workspace_size_grows_with_batch():
    a = mla.workspace_size(128, 1, 4096, mla.MLA_BF16, mla.MLA_BF16)
    b = mla.workspace_size(128, 64, 4096, mla.MLA_BF16, mla.MLA_BF16)
    assert 0 < a < b and b % 256 == 0
    assert mla.workspace_size(128, 0, 4096, mla.MLA_BF16, mla.MLA_BF16) > 0
    bad = mla.Dims(128, 256, 64, 128, 128)
    assert mla.load().mla_decode_workspace_size(ctypes.byref(bad), 1, 16, 1, 1, None) == 0


def _decode_status(dims, act=mla.MLA_BF16, cdt=mla.MLA_BF16, batch=1, max_len=16, ptr=16,
                   ls=576, rs=576, rows=64, cap=16, ws=1 << 20, scale=0.07, scales=True):
    lib = mla.load()
    p = ctypes.c_void_p(ptr) if ptr else None
    sc = p if scales else None
    return lib.mla_decode(ctypes.byref(dims), p, p, p, p, act, p, ls, p, rs, sc, cdt, rows, cap,
                          p, batch, max_len, scale, p, None, p, ws, None, None)


def test_decode_argument_errors():
    d = mla.dims(128)
    assert _decode_status(d, batch=0) == 0                            # no-op
    assert _decode_status(d, ptr=0) == 1                              # null pointers
    assert _decode_status(d, batch=-1) == 1
    assert _decode_status(d, ls=500) == 1                             # stride < 512
    assert _decode_status(d, ls=577) == 1                             # misaligned rows
    assert _decode_status(d, ptr=8) == 1                              # misaligned pointers
    assert _decode_status(d, cap=8) == 1                              # capacity < max_len
    assert _decode_status(d, rows=8) == 1                             # rows < batch * capacity
    assert _decode_status(d, scale=float("nan")) == 1
    assert _decode_status(mla.dims(48)) == 2                          # heads % 32
    assert _decode_status(mla.Dims(128, 512, 64, 128, 64)) == 2       # d_v
    assert _decode_status(d, act=mla.MLA_F32, cdt=mla.MLA_BF16) == 2  # dtype combination
    assert _decode_status(d, cdt=mla.MLA_FP8_E4M3, scales=False) == 1  # fp8 without scales
    assert _decode_status(d, ws=16) == 3                              # workspace too small


def test_paged_and_append_argument_errors():
    lib = mla.load()
    d = mla.dims(128)
    p = ctypes.c_void_p(16)
    # block_size must be a positive multiple of 32; table must cover max_len
    for bs, mb, ml in ((48, 4, 64), (0, 4, 64), (64, 1, 100)):
        st = lib.mla_decode_paged(ctypes.byref(d), p, p, p, p, 1, p, 576, p, 576, None, 1, 1024,
                                  p, mb, bs, p, 1, ml, 0.07, p, None, p, 1 << 20, None, None)
        assert st == 1, (bs, mb, ml)
    # append: bad theta, unsupported input dtype, null positions
    args = [ctypes.byref(d), p, p, 1, p, 1, p, 576, p, 576, None, 1, 64, 64, None, 0, 64]
    assert lib.mla_cache_append(*args, -1.0, None) == 1
    bad_in = list(args)
    bad_in[3] = 2
    assert lib.mla_cache_append(*bad_in, 10000.0, None) == 2
    no_pos = list(args)
    no_pos[4] = None
    assert lib.mla_cache_append(*no_pos, 10000.0, None) == 1
    zero = list(args)
    zero[5] = 0
    assert lib.mla_cache_append(*zero, 10000.0, None) == 0


def test_project_argument_errors():
    lib = mla.load()
    d = mla.dims(128)
    p = ctypes.c_void_p(16)
    assert lib.mla_project_workspace_size(64, 7168) >= 64 * 576 * 4
    assert lib.mla_project_workspace_size(64, 100) == 0        # d_model not a multiple of 64
    assert lib.mla_project_workspace_size(-1, 7168) == 0

    def call(d_model=7168, batch=4, act=1, w_kr=p, ws=p, ws_bytes=1 << 30, theta=10000.0):
        return lib.mla_project_append(ctypes.byref(d), p, p, w_kr, act, d_model, p, batch, p, 576,
                                      p, 576, None, 1, 4096, 1024, None, 0, 64, theta, ws,
                                      ws_bytes, None)
    assert call(d_model=100) == 1
    assert call(d_model=0) == 1
    assert call(w_kr=None) == 1
    assert call(act=2) == 2                                       # fp8 activations
    assert call(theta=-1.0) == 1
    assert call(ws=None) == 3
    assert call(ws_bytes=1024) == 3
    assert call(batch=0) == 0


def test_projected_append_argument_errors():
    """A decode call whose append takes a projection workspace checks its
    d_model (a positive multiple of 64) before launching anything; mla_project
    checks its sizes and workspace like mla_project_append."""
    lib = mla.load()
    d = mla.dims(128)
    p = ctypes.c_void_p(16)
    for d_model in (0, 100):
        a = mla.AppendArgs(None, None, mla.MLA_F32, 16, 10000.0, 16, d_model)
        o = mla.DecodeOptions()
        o.append = ctypes.pointer(a)
        st = lib.mla_decode(ctypes.byref(d), p, p, p, p, 1, p, 576, p, 576, None, 1, 4096, 1024,
                            p, 4, 1024, 0.07, p, None, p, 1 << 30, ctypes.byref(o), None)
        assert st == 1, (d_model, st)
    assert lib.mla_project(ctypes.byref(d), p, p, p, 1, 100, 4, p, 1 << 30, None) == 1
    assert lib.mla_project(ctypes.byref(d), p, p, None, 1, 7168, 4, p, 1 << 30, None) == 1
    assert lib.mla_project(ctypes.byref(d), p, p, p, 2, 7168, 4, p, 1 << 30, None) == 2
    assert lib.mla_project(ctypes.byref(d), p, p, p, 1, 7168, 4, p, 1024, None) == 3
    assert lib.mla_project(ctypes.byref(d), p, p, p, 1, 7168, 0, p, 0, None) == 0
