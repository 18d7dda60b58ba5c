"""CPU oracle for Multi-Head Latent Attention (MLA) decode: TEST INFRASTRUCTURE ONLY.

This is a plain, slow, deliberately unoptimised float64 reference that the test
suite, the smoke check and the benchmark's CPU-baseline leg compare the HIP
library against. Nothing in the product path may import it. It shares no code
with the HIP library: its number-format decoders, its rounding, its RoPE and
its block-table gather are written here from their definitions.

Sources, cited by page title and section:

* [WL] "How DeepSeek Rewrote the Transformer [MLA]" (linuxpro.com.br, English
  edition), sections "Classic attention and the cost of the KV cache",
  "MLA: compress the pair, not the heads".
* [TN] "DeepSeek AI efficiency, architecture, benchmarks" (technova-ai.online),
  section "Architectural Innovations: Multi-Head Latent Attention (MLA)",
  equations for c_KV, K_t and V_t.
* [IA] "Como a MLA da DeepSeek cortou 93% da memoria ..." (ia.com.br), sections
  "Um resumo no lugar de 128 copias" and "A conta feita fora da DeepSeek".
* [KV] "How Transformers Become Faster And Smarter: From KV Cache to MLA",
  sections "Decoder Inference" and "KV Cache" (the causal-mask experiment).

Readings taken where the pages are silent (each is listed again in the design
notes):

* W_UK[h] is stored [d_nope, d_c] and maps a latent row to a key (column
  convention of [TN]: K = W_UK c), so the absorbed query is q_nope . W_UK[h].
  W_UV[h] is stored [d_c, d_v] and maps a latent row to a value (row convention
  v = c W_UV[h]).
* The decoupled RoPE key k_pe (64 wide) is one per token and shared by all
  heads ([WL] "MLA: compress the pair, not the heads": the cache does not
  depend on the head count); q_pe is per head; a score is the sum of the two
  dot products, scaled by 1/sqrt(d_nope + d_rope).
* The causal mask of a single decode query is the length mask: rows
  0 .. len-1 exist, the rest are excluded exactly (not by a large negative
  number).
* RoPE: base 10000, interleaved pairs (2i, 2i+1), angle p * base^(-2i/d_rope)
  at 0-based position p.
* fp8 cache: OCP e4m3fn codes, one bf16 scale per token row covering all 576
  values; scale = bf16_rne(amax / 448) computed in fp32 (1 when amax == 0);
  code = e4m3fn_rne_saturating(x / scale) with the division in fp32. The
  quantiser takes its integer decisions in fp32, the precision of the kernel.

Functions whose result has no independent pin are marked "parity unpinned";
at present there are none (see tests/test_oracle_*.py for the pins).
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats, from their definitions
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen by 16 zero bits."""
    u16 = np.asarray(bits).astype(np.uint16)
    u32 = u16.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits).astype(np.uint32).view(np.float32).astype(np.float64)


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ('fn': no infinities, only S.1111.111 is NaN), bias 7.

    normal   (e > 0): (-1)^s * 2^(e-7) * (1 + m/8)
    subnormal(e = 0): (-1)^s * 2^(-6) * (m/8)
    """
    b = np.asarray(bits).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def _round_rne(x: np.ndarray, mant_bits: int, emin: int) -> np.ndarray:
    """Round float64 values to a binary format with `mant_bits` stored mantissa
    bits and minimum normal exponent `emin`, round-to-nearest, ties to even.
    No overflow handling (callers saturate or check range)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    # exponent of the leading bit, exactly (frexp gives ax = f * 2^fe, f in [0.5, 1))
    _, fe = np.frexp(np.where(ax > 0, ax, 1.0))
    e = (fe - 1).astype(np.int64)
    e = np.maximum(e, emin)
    quantum = np.ldexp(1.0, e - mant_bits)
    q = ax / quantum  # exact: power-of-two scaling
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))
    r = r + up
    return np.sign(x) * r * quantum


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (7 stored mantissa bits, emin -126), ties to even."""
    return _round_rne(x, 7, -126)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


E4M3_MAX = 448.0


def round_to_e4m3fn_sat(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn value (3 mantissa bits, emin -6), ties to even, then
    clamped to +-448 (the largest finite code)."""
    r = _round_rne(x, 3, -6)
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def e4m3fn_value_to_bits(v: np.ndarray) -> np.ndarray:
    """Encode exactly representable e4m3fn values into their 8-bit codes."""
    v = np.asarray(v, dtype=np.float64)
    s = (np.signbit(v)).astype(np.int64)
    a = np.abs(v)
    _, fe = np.frexp(np.where(a > 0, a, 1.0))
    e_unb = fe - 1
    is_norm = (a >= 2.0 ** -6)
    e_field = np.where(is_norm, e_unb + 7, 0)
    m_field = np.where(is_norm, np.round((a / np.ldexp(1.0, e_unb) - 1.0) * 8.0),
                       np.round(a / 2.0 ** -9))
    m_field = np.where(a == 0, 0, m_field).astype(np.int64)
    e_field = np.where(a == 0, 0, e_field).astype(np.int64)
    return ((s << 7) | (e_field << 3) | m_field).astype(np.uint8)


def bf16_value_to_bits(v: np.ndarray) -> np.ndarray:
    """Encode exactly representable bfloat16 values into their 16-bit codes."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# the value of every e4m3fn code, from the definition above (one entry per
# code), so that large caches decode by table lookup
_E4M3FN_TABLE = e4m3fn_bits_to_f64(np.arange(256))


def decode_storage(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage (uint16 for bf16, uint32 for f32, uint8 for e4m3) -> float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f32":
        return f32_bits_to_f64(bits)
    if dtype == "fp8":
        return _E4M3FN_TABLE[np.asarray(bits).astype(np.uint8)]
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# RoPE on the decoupled key ([WL] "MLA: compress the pair, not the heads": the
# 64-wide k^R is cached beside the latent; formula not given -> reading above)
# ---------------------------------------------------------------------------

ROPE_BASE = 10000.0


def rope_angles(pos: int, d_rope: int, base: float = ROPE_BASE) -> np.ndarray:
    i = np.arange(d_rope // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d_rope)
    return float(pos) * theta


def rope_rotate(x: np.ndarray, pos: int, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate interleaved pairs (x[2i], x[2i+1]) by angle pos*theta_i."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, base)
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# ---------------------------------------------------------------------------
# Cache addressing (integer work; must match the library bit for bit)
# ---------------------------------------------------------------------------


def contiguous_row(b: int, t: int, seq_capacity: int) -> int:
    """Row of token t of sequence b in a contiguous cache of seq_capacity rows
    per sequence."""
    return b * seq_capacity + t


def paged_row(block_table: np.ndarray, b: int, t: int, block_size: int) -> int:
    """Row of token t of sequence b in a paged pool: block_table[b][t // bs]
    names the physical block, t % bs the slot inside it."""
    blk = int(block_table[b][t // block_size])
    return blk * block_size + (t % block_size)


def gather_rows(b: int, n: int, *, seq_capacity=None, block_table=None,
                block_size=None) -> np.ndarray:
    """Physical row index of tokens 0..n-1 of sequence b: the two formulas
    above, evaluated for all t at once."""
    t = np.arange(n, dtype=np.int64)
    if block_table is None:
        return b * int(seq_capacity) + t
    blocks = np.asarray(block_table)[b].astype(np.int64)
    return blocks[t // block_size] * block_size + t % block_size


# ---------------------------------------------------------------------------
# Attention, non-absorbed (the definition) and absorbed (the identity of [WL]
# "MLA: compress the pair, not the heads": Q K^T = (Q W_UK^T) c^T)
# ---------------------------------------------------------------------------


def softmax_attend(scores: np.ndarray, values: np.ndarray):
    """Plain softmax over the last axis of `scores` [n], weights . values [n, d].
    Returns (output [d], lse) with lse = natural log of sum exp(scores).
    n == 0 yields zeros and -inf (empty attention)."""
    n = scores.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -math.inf
    m = np.max(scores)
    e = np.exp(scores - m)
    l = np.sum(e)
    p = e / l
    return p @ values, m + math.log(l)


def decode_head_nonabsorbed(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
    """One head of MLA decode in the non-absorbed form.

    [TN] "Architectural Innovations: MLA": K_t = W_UK c_KV, V_t = W_UV c_KV;
    [WL] "Classic attention ...": softmax(Q K^T / sqrt(d_k) + M) V, with the
    decoupled RoPE key appended to every key ([WL] "MLA: compress the pair").

    q_nope [d_nope], q_pe [d_rope], w_uk_h [d_nope, d_c], w_uv_h [d_c, d_v],
    C [n, d_c] latent rows, R [n, d_rope] rotated RoPE keys.
    """
    K = C @ w_uk_h.T          # [n, d_nope]: each key k_t = W_UK[h] c_t
    V = C @ w_uv_h            # [n, d_v]:    each value v_t = c_t W_UV[h]
    s = scale * (K @ q_nope + R @ q_pe)
    return softmax_attend(s, V)


def decode_head_absorbed(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
    """Same head computed by associativity: the query is absorbed into latent
    space (q_lat = q_nope W_UK[h]) and W_UV[h] is applied after mixing the
    latent rows ([WL] "MLA: compress the pair, not the heads")."""
    q_lat = q_nope @ w_uk_h   # [d_c]
    s = scale * (C @ q_lat + R @ q_pe)
    o_lat, lse = softmax_attend(s, C)
    return o_lat @ w_uv_h, lse


def decode(q_nope, q_pe, w_uk, w_uv, latent_rows, rope_rows, scale, *,
           heads=None, absorbed=False):
    """Batched MLA decode.

    q_nope [B, H, d_nope], q_pe [B, H, d_rope] (already rotated),
    w_uk [H, d_nope, d_c], w_uv [H, d_c, d_v],
    latent_rows: list of B arrays [N_b, d_c]; rope_rows: list of B arrays
    [N_b, d_rope] (the gathered, dequantised cache of each sequence).
    Returns out [B, H, d_v] and lse [B, H] (natural log; -inf for N_b = 0).
    `heads` restricts the computation to a subset (others are left NaN).
    """
    B, H, _ = q_nope.shape
    d_v = w_uv.shape[2]
    out = np.full((B, H, d_v), np.nan)
    lse = np.full((B, H), np.nan)
    hs = range(H) if heads is None else heads
    fn = decode_head_absorbed if absorbed else decode_head_nonabsorbed
    for b in range(B):
        C = latent_rows[b]
        R = rope_rows[b]
        for h in hs:
            out[b, h], lse[b, h] = fn(q_nope[b, h], q_pe[b, h], w_uk[h], w_uv[h],
                                      C, R, scale)
    return out, lse


def decode_seq_absorbed(q_nope, q_pe, w_uk, w_uv, C, R, scale):
    """Every head of one sequence in the absorbed form, the same sums as
    decode_head_absorbed written as matrix products over the head axis:
    q_lat[h] = q_nope[h] W_UK[h]; S[t, h] = scale (c_t . q_lat[h] + k^R_t .
    q_pe[h]); softmax over t for each h; o[h] = (sum_t P[t, h] c_t) W_UV[h].

    q_nope [H, d_nope], q_pe [H, d_rope], w_uk [H, d_nope, d_c],
    w_uv [H, d_c, d_v], C [n, d_c], R [n, d_rope].
    Returns out [H, d_v] and lse [H] (zeros and -inf when n == 0)."""
    H = q_nope.shape[0]
    n = C.shape[0]
    if n == 0:
        return np.zeros((H, w_uv.shape[2])), np.full(H, -math.inf)
    q_lat = np.einsum("hk,hkc->hc", q_nope, w_uk)       # [H, d_c]
    S = scale * (C @ q_lat.T + R @ q_pe.T)              # [n, H]
    m = S.max(axis=0)
    E = np.exp(S - m)
    l = E.sum(axis=0)
    P = E / l
    o_lat = P.T @ C                                     # [H, d_c]
    return np.einsum("hc,hcv->hv", o_lat, w_uv), m + np.log(l)


def decode_model_io(x, q_pe, w_q, w_uk, w_uv, w_o, C, R, scale):
    """Decode of one token from its model-width input to its model-width
    output, unfused (the definition): q_nope[h] = W_Q[h] x (column
    convention of [TN]'s projections; W_Q[h] is [d_nope, d_model]), each
    head's attention over the cache as in decode_head_nonabsorbed, then the
    output projection y = sum_h o[h] W_O[h] (W_O[h] is [d_v, d_model]: head
    h's rows of the output matrix W_O that [WL] "MLA: compress the pair, not
    the heads" names).

    x [d_model], q_pe [H, d_rope] (already rotated), C [n, d_c], R [n, d_rope].
    Returns y [d_model] and lse [H]."""
    H = w_q.shape[0]
    y = np.zeros(w_o.shape[2])
    lse = np.empty(H)
    for h in range(H):
        q_nope = w_q[h] @ x
        o, lse[h] = decode_head_nonabsorbed(q_nope, q_pe[h], w_uk[h], w_uv[h], C, R, scale)
        y += o @ w_o[h]
    return y, lse


def fuse_query_weight(w_q_h, w_uk_h):
    """W_UK absorbed into the query projection, offline ([WL] "MLA: compress
    the pair, not the heads": absorb W_UK into the Q matrix before serving):
    q_lat = q_nope W_UK[h] = (W_Q[h] x)^T W_UK[h], so q_lat = W_QK[h] x with
    W_QK[h] = W_UK[h]^T W_Q[h], [d_c, d_model]."""
    return w_uk_h.T @ w_q_h


def fuse_output_weight(w_uv_h, w_o_h):
    """W_UV absorbed into the output matrix, offline (same passage: W_UV goes
    into W_O): o W_O[h] = (o_lat W_UV[h]) W_O[h] = o_lat W_VO[h] with
    W_VO[h] = W_UV[h] W_O[h], [d_c, d_model]."""
    return w_uv_h @ w_o_h


def decode_model_io_fused(x, q_pe, w_qk, w_vo, C, R, scale):
    """The same decode with the fused weights: every head scores its absorbed
    query W_QK[h] x against the latent rows, mixes them, and the mixed latent
    goes through W_VO[h] straight to the model width.
    Returns y [d_model] and lse [H]."""
    H = w_qk.shape[0]
    y = np.zeros(w_vo.shape[2])
    lse = np.empty(H)
    for h in range(H):
        q_lat = w_qk[h] @ x
        s = scale * (C @ q_lat + R @ q_pe[h])
        o_lat, lse[h] = softmax_attend(s, C)
        y += o_lat @ w_vo[h]
    return y, lse


def causal_prefill(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
    """Full causal self-attention of T queries over T cached rows for one head:
    row t attends to rows 0..t ([KV] "KV Cache": the causal mask hides the
    future). Returns out [T, d_v]. Written in matrix form with an exact mask."""
    K = C @ w_uk_h.T
    V = C @ w_uv_h
    S = scale * (q_nope @ K.T + q_pe @ R.T)    # [T, T]
    T = S.shape[0]
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    S = np.where(mask, -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    P = E / E.sum(axis=1, keepdims=True)
    return P @ V


def chunked_prefill(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
    """One head of prefill over a chunk of T new queries whose rows are the
    last T of the n cached rows (n >= T, the context before the chunk being
    the first n - T rows): query i sits at position n - T + i and attends to
    rows 0 .. n - T + i ([WL] "Classic attention and the cost of the KV
    cache": softmax(Q K^T / sqrt(d_k) + M) V with the causal mask M; [KV]
    "KV Cache": each token sees itself and the tokens before it).

    Recompute (non-absorbed) form: every key k_t = [W_UK[h] c_t ; k^R_t] and
    value v_t = c_t W_UV[h] is decompressed from the latent rows ([TN]
    equations for K and V), then plain causal softmax attention.
    q_nope [T, d_nope], q_pe [T, d_rope], C [n, d_c], R [n, d_rope].
    Returns out [T, d_v] and lse [T] (natural log). When n < T the first
    T - n queries sit before position 0 and see no row: their attention is
    empty (zeros and -inf, as for an empty sequence in decode)."""
    T = q_nope.shape[0]
    n = C.shape[0]
    K = C @ w_uk_h.T                                  # [n, d_nope]
    V = C @ w_uv_h                                    # [n, d_v]
    S = scale * (q_nope @ K.T + q_pe @ R.T)           # [T, n]
    pos = (n - T) + np.arange(T)
    S = np.where(np.arange(n)[None, :] > pos[:, None], -np.inf, S)
    out = np.zeros((T, w_uv_h.shape[1]))
    lse = np.full(T, -math.inf)
    seen = pos >= 0                                   # queries with at least row 0
    if np.any(seen):
        Ss = S[seen]
        m = Ss.max(axis=1, keepdims=True)
        E = np.exp(Ss - m)
        l = E.sum(axis=1, keepdims=True)
        out[seen] = (E / l) @ V
        lse[seen] = (m + np.log(l))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# Cache append (write the new token's row)
# ---------------------------------------------------------------------------


FP32_MIN_NORMAL = 2.0 ** -126


def fp8_row_scale(row32: np.ndarray) -> float:
    """Per-token scale of an fp8 row (values given in fp32):
    amax == 0 -> 1; amax/448 (fp32 division) below the smallest normal fp32
    -> 2^-126; otherwise the nearest bf16 of amax/448 (ties to even)."""
    amax = np.float32(np.max(np.abs(row32)))
    if amax == 0:
        return 1.0
    s32 = np.float32(amax / np.float32(E4M3_MAX))
    if float(s32) < FP32_MIN_NORMAL:
        return FP32_MIN_NORMAL
    return float(round_to_bf16(np.float64(s32)))


def append_row(c_kv: np.ndarray, k_pe: np.ndarray, pos: int, cache_dtype: str):
    """Row written for one token: latent c_t copied (rounded to the cache
    type) and k_pe rotated by RoPE at position `pos` ([WL] "MLA: compress the
    pair, not the heads": both go to the cache, 576 numbers).

    c_kv, k_pe: float64 values of the inputs (already decoded).
    Returns (latent_values, rope_values, scale or None, codes or None):
      bf16/f32 caches: the rounded values (float64), scale None;
      fp8 cache: dequantised values, the bf16 scale value, and the 8-bit codes.
    """
    rot = rope_rotate(k_pe, pos)
    if cache_dtype == "f32":
        return round_to_f32(c_kv), round_to_f32(rot), None, None
    if cache_dtype == "bf16":
        return round_to_bf16(c_kv), round_to_bf16(rot), None, None
    if cache_dtype != "fp8":
        raise ValueError(cache_dtype)
    # fp8: the kernel holds the row in fp32 (inputs are exact in fp32, the
    # rotation is rounded to fp32), so the quantiser is emulated in fp32.
    row32 = np.concatenate([c_kv, rot]).astype(np.float32)
    scale = fp8_row_scale(row32)
    q32 = (row32 / np.float32(scale)).astype(np.float32)
    vals = round_to_e4m3fn_sat(q32.astype(np.float64))
    codes = e4m3fn_value_to_bits(vals)
    deq = vals * scale
    d_c = c_kv.shape[0]
    return deq[:d_c], deq[d_c:], scale, codes


# ---------------------------------------------------------------------------
# Down-projection of the new token ([TN] "Architectural Innovations:
# Multi-Head Latent Attention (MLA)", equation for c_KV; [WL] "MLA: compress
# the pair, not the heads", diagram: the input h_t gives both the 512-wide
# latent and the 64-wide RoPE key that go to the cache)
# ---------------------------------------------------------------------------


def kv_down_project(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray):
    """Latent c_KV = W_DKV h and un-rotated RoPE key W_KR h of one token.

    Column convention of the [TN] equation: W_DKV is [d_c, d_model] and W_KR
    [d_rope, d_model] (reading: the pages name the RoPE key's projection only
    through the diagram, so it takes the same convention), h is [d_model].
    float64 products, no bias and no normalisation (the pages give neither).
    """
    return w_dkv @ h, w_kr @ h


def project_append_row(h, w_dkv, w_kr, pos: int, cache_dtype: str):
    """Row written for a token given its hidden state: the down-projection,
    then the append of the latent and the RoPE-rotated key (append_row)."""
    c, k = kv_down_project(h, w_dkv, w_kr)
    return append_row(c, k, pos, cache_dtype)


# ---------------------------------------------------------------------------
# Cache-size closed forms ([WL] "Classic attention and the cost of the KV
# cache" and "MLA: compress the pair, not the heads"; [IA] "A conta feita
# fora da DeepSeek")
# ---------------------------------------------------------------------------


def mha_cache_bytes_per_token(d_h: int, n_heads: int, layers: int, elem_bytes: int) -> int:
    """2 (K and V) x d_h x n_heads x L x bytes, per token."""
    return 2 * d_h * n_heads * layers * elem_bytes


def mla_cache_bytes_per_token(d_c: int, d_rope: int, layers: int, elem_bytes: int,
                              scale_bytes: int = 0) -> int:
    """(latent + RoPE key) x bytes (+ per-row scale) x L, per token."""
    return ((d_c + d_rope) * elem_bytes + scale_bytes) * layers


def gqa_equivalent_groups(d_c: int, d_rope: int, d_h: int) -> float:
    """Number of K/V head pairs whose cache equals one MLA row."""
    return (d_c + d_rope) / (2.0 * d_h)
