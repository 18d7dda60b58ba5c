"""Python binding of the MI355X MLA decode library (ctypes over libmla_hip.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/mla.h. PyTorch supplies device
memory (tensors) and the current HIP stream. There is no fallback: if the
library is missing, every entry point raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_hip.so")

MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
D_C, D_ROPE, D_NOPE, D_V = 512, 64, 128, 128

SYMBOLS = ("mla_status_string", "mla_cache_bytes_per_token", "mla_cache_append",
           "mla_decode_workspace_size", "mla_decode", "mla_decode_paged",
           "mla_project_append", "mla_project_workspace_size", "mla_project")


class MLAError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{text} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32)]


class AppendArgs(ctypes.Structure):
    _fields_ = [("c_kv", ctypes.c_void_p), ("k_pe", ctypes.c_void_p), ("in_dtype", ctypes.c_int),
                ("positions", ctypes.c_void_p), ("rope_theta", ctypes.c_float),
                ("projected", ctypes.c_void_p), ("d_model", ctypes.c_int32)]


class DecodeOptions(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("attn_begin", ctypes.c_void_p), ("attn_end", ctypes.c_void_p),
                ("append", ctypes.POINTER(AppendArgs))]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"MLA HIP library not built: {p} is missing "
                           "(run head_latent_attention_07_amd/build.py)")
    lib = ctypes.CDLL(p)
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_cache_bytes_per_token.restype = _SZ
    lib.mla_cache_bytes_per_token.argtypes = [ctypes.c_int, _I32, _I32]
    lib.mla_decode_workspace_size.restype = _SZ
    lib.mla_decode_workspace_size.argtypes = [ctypes.POINTER(Dims), _I32, _I32, ctypes.c_int,
                                              ctypes.c_int, ctypes.POINTER(DecodeOptions)]
    lib.mla_cache_append.restype = ctypes.c_int
    lib.mla_cache_append.argtypes = [ctypes.POINTER(Dims), _P, _P, ctypes.c_int, _P, _I32,
                                     _P, _I64, _P, _I64, _P, ctypes.c_int, _I64, _I64, _P, _I32,
                                     _I32, _F, _P]
    common = [ctypes.POINTER(Dims), _P, _P, _P, _P, ctypes.c_int, _P, _I64, _P, _I64, _P,
              ctypes.c_int, _I64]
    tail = [_P, _I32, _I32, _F, _P, _P, _P, _SZ, ctypes.POINTER(DecodeOptions), _P]
    lib.mla_decode.restype = ctypes.c_int
    lib.mla_decode.argtypes = common + [_I64] + tail
    lib.mla_decode_paged.restype = ctypes.c_int
    lib.mla_decode_paged.argtypes = common + [_P, _I32, _I32] + tail
    lib.mla_project_workspace_size.restype = _SZ
    lib.mla_project_workspace_size.argtypes = [_I32, _I32]
    lib.mla_project.restype = ctypes.c_int
    lib.mla_project.argtypes = [ctypes.POINTER(Dims), _P, _P, _P, ctypes.c_int, _I32, _I32, _P, _SZ,
                                _P]
    lib.mla_project_append.restype = ctypes.c_int
    lib.mla_project_append.argtypes = [ctypes.POINTER(Dims), _P, _P, _P, ctypes.c_int, _I32, _P,
                                       _I32, _P, _I64, _P, _I64, _P, ctypes.c_int, _I64, _I64, _P,
                                       _I32, _I32, _F, _P, _SZ, _P]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise MLAError(status, load().mla_status_string(status).decode())


def status_string(status: int) -> str:
    return load().mla_status_string(status).decode()


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MLA_F32
    if t == torch.bfloat16:
        return MLA_BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return MLA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t}")


def cache_bytes_per_token(cache_dtype: int, d_c: int = D_C, d_rope: int = D_ROPE) -> int:
    return int(load().mla_cache_bytes_per_token(cache_dtype, d_c, d_rope))


def dims(heads: int) -> Dims:
    return Dims(heads, D_C, D_ROPE, D_NOPE, D_V)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _opts(num_splits: int = 0, events: Optional[Tuple[int, int]] = None, append=None):
    """mla_decode_options for the call (None when every field is a default).
    `append` = (c_kv, k_pe, positions[, rope_theta]) appends those rows first;
    (None, None, positions, rope_theta, workspace, d_model) appends the rows of
    a preceding project() call whose workspace that is."""
    if not num_splits and events is None and append is None:
        return None
    o = DecodeOptions()
    o.num_splits = num_splits
    if events is not None:
        o.attn_begin, o.attn_end = events
    if append is not None:
        c_kv, k_pe, positions = append[:3]
        theta = append[3] if len(append) > 3 else 10000.0
        if len(append) > 4:          # rows from a projection workspace
            a = AppendArgs(None, None, MLA_F32, _ptr(positions), theta, _ptr(append[4]),
                           int(append[5]))
        else:
            a = AppendArgs(_ptr(c_kv), _ptr(k_pe), dtype_code(c_kv.dtype), _ptr(positions), theta,
                           None, 0)
        o._append_keep = a            # the struct must outlive the call
        o.append = ctypes.pointer(a)
    return ctypes.byref(o)


def workspace_size(heads: int, batch: int, max_len: int, act_dtype: int, cache_dtype: int,
                   num_splits: int = 0) -> int:
    d = dims(heads)
    return int(load().mla_decode_workspace_size(ctypes.byref(d), batch, max_len, act_dtype,
                                                cache_dtype, _opts(num_splits)))


def split_cache(cache: torch.Tensor):
    """Latent and RoPE-key views of a packed [rows, 576] cache."""
    return cache[:, :D_C], cache[:, D_C:]


def cache_append(c_kv: torch.Tensor, k_pe: torch.Tensor, positions: torch.Tensor,
                 latent: torch.Tensor, rope: torch.Tensor, *, heads: int,
                 scales: Optional[torch.Tensor] = None, seq_capacity: int = 0,
                 block_table: Optional[torch.Tensor] = None, block_size: int = 64,
                 rope_theta: float = 10000.0, stream=None) -> None:
    """Write the new tokens' latent rows and RoPE-rotated keys (mla_cache_append)."""
    lib = load()
    d = dims(heads)
    B = c_kv.shape[0]
    max_blocks = 0 if block_table is None else block_table.shape[1]
    _check(lib.mla_cache_append(
        ctypes.byref(d), _ptr(c_kv), _ptr(k_pe), dtype_code(c_kv.dtype), _ptr(positions), B,
        _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0), _ptr(scales),
        dtype_code(latent.dtype), latent.shape[0], seq_capacity, _ptr(block_table), max_blocks,
        block_size, rope_theta, _stream(stream)))


def project_workspace_size(batch: int, d_model: int) -> int:
    return int(load().mla_project_workspace_size(batch, d_model))


def project_append(hidden: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor,
                   positions: torch.Tensor, latent: torch.Tensor, rope: torch.Tensor, *,
                   heads: int, scales: Optional[torch.Tensor] = None, seq_capacity: int = 0,
                   block_table: Optional[torch.Tensor] = None, block_size: int = 64,
                   rope_theta: float = 10000.0, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Project the new tokens' hidden states to their latent rows and RoPE keys
    and append them (mla_project_append)."""
    lib = load()
    d = dims(heads)
    B, D = hidden.shape
    if workspace is None:
        workspace = torch.empty(project_workspace_size(B, D), dtype=torch.uint8,
                                device=hidden.device)
    max_blocks = 0 if block_table is None else block_table.shape[1]
    _check(lib.mla_project_append(
        ctypes.byref(d), _ptr(hidden), _ptr(w_dkv), _ptr(w_kr), dtype_code(hidden.dtype), D,
        _ptr(positions), B, _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0),
        _ptr(scales), dtype_code(latent.dtype), latent.shape[0], seq_capacity, _ptr(block_table),
        max_blocks, block_size, rope_theta, _ptr(workspace), workspace.numel(), _stream(stream)))


def project(hidden: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor,
            workspace: torch.Tensor, *, heads: int = 128, stream=None) -> None:
    """The down-projection alone (mla_project): partial sums of the new rows
    left in `workspace` for a following decode call's append."""
    B, D = hidden.shape
    _check(load().mla_project(ctypes.byref(dims(heads)), _ptr(hidden), _ptr(w_dkv), _ptr(w_kr),
                              dtype_code(hidden.dtype), D, B, _ptr(workspace), workspace.numel(),
                              _stream(stream)))


def _decode(paged: bool, q_nope, q_pe, w_uk, w_uv, latent, rope, lengths, max_len, *,
            scales=None, seq_capacity=0, block_table=None, block_size=64, softmax_scale=None,
            out=None, lse=None, workspace=None, num_splits=0, events=None, append=None,
            stream=None, want_lse=True):
    lib = load()
    B, H = q_nope.shape[0], q_nope.shape[1]
    d = dims(H)
    act = dtype_code(q_nope.dtype)
    cdt = dtype_code(latent.dtype)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D_NOPE + D_ROPE)
    dev = q_nope.device
    if out is None:
        out = torch.empty((B, H, D_V), dtype=q_nope.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if workspace is None:
        ws = workspace_size(H, B, max_len, act, cdt, num_splits)
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    opts = _opts(num_splits, events, append)
    head = [ctypes.byref(d), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv), act,
            _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0), _ptr(scales), cdt,
            latent.shape[0]]
    tail = [_ptr(lengths), B, max_len, softmax_scale, _ptr(out), _ptr(lse), _ptr(workspace),
            workspace.numel(), opts, _stream(stream)]
    if paged:
        st = lib.mla_decode_paged(*head, _ptr(block_table), block_table.shape[1], block_size, *tail)
    else:
        st = lib.mla_decode(*head, seq_capacity, *tail)
    _check(st)
    return out, lse


def decode(q_nope, q_pe, w_uk, w_uv, latent, rope, lengths, max_len, *, seq_capacity, **kw):
    """MLA decode over a contiguous cache (mla_decode). Returns (out, lse)."""
    return _decode(False, q_nope, q_pe, w_uk, w_uv, latent, rope, lengths, max_len,
                   seq_capacity=seq_capacity, **kw)


def decode_paged(q_nope, q_pe, w_uk, w_uv, latent, rope, lengths, max_len, *, block_table,
                 block_size=64, **kw):
    """MLA decode over a paged cache (mla_decode_paged). Returns (out, lse)."""
    return _decode(True, q_nope, q_pe, w_uk, w_uv, latent, rope, lengths, max_len,
                   block_table=block_table, block_size=block_size, **kw)


def decode_inputs(inp, **kw):
    """Run the decode entry point matching a synthetic workload (see synth)."""
    lat, rop = split_cache(inp.cache)
    if inp.paged:
        return decode_paged(inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, lat, rop, inp.lengths,
                            inp.max_len, block_table=inp.block_table, block_size=inp.block_size,
                            scales=inp.scales, softmax_scale=inp.scale, **kw)
    return decode(inp.q_nope, inp.q_pe, inp.w_uk, inp.w_uv, lat, rop, inp.lengths, inp.max_len,
                  seq_capacity=inp.seq_capacity, scales=inp.scales, softmax_scale=inp.scale, **kw)
