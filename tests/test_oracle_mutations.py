"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
its pins catch every one of them: a pin set that passes a broken oracle pins
nothing."""

import importlib.util
import math
import os

import numpy as np
import pytest

import oracle_pins as P

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "mla_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("mla_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_drop_rope_term(o):
    def f(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
        K = C @ w_uk_h.T
        return o.softmax_attend(scale * (K @ q_nope), C @ w_uv_h)
    o.decode_head_nonabsorbed = f


def m_wrong_scale(o):
    orig = o.decode_head_nonabsorbed
    o.decode_head_nonabsorbed = lambda *a: orig(*a[:-1], a[-1] * math.sqrt(2.0))


def m_head_index(o):
    orig = o.decode

    def f(q_nope, q_pe, w_uk, w_uv, lat, rope, scale, **kw):
        return orig(q_nope, q_pe, np.repeat(w_uk[:1], w_uk.shape[0], 0), w_uv, lat, rope, scale, **kw)
    o.decode = f


def m_uv_for_uk_layout(o):
    # use the absorbed latent output without W_UV's proper contraction axis
    def f(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
        K = C @ w_uk_h.T
        V = C @ (w_uv_h[::-1])
        return o.softmax_attend(scale * (K @ q_nope + R @ q_pe), V)
    o.decode_head_nonabsorbed = f


def m_unnormalised(o):
    def f(scores, values):
        m = np.max(scores) if len(scores) else 0.0
        e = np.exp(scores - m)
        return e @ values, m + math.log(np.sum(e)) if len(scores) else -math.inf
    o.softmax_attend = f


def m_lse_without_max(o):
    def f(scores, values):
        if len(scores) == 0:
            return np.zeros(values.shape[1]), -math.inf
        m = np.max(scores)
        e = np.exp(scores - m)
        return (e / e.sum()) @ values, math.log(e.sum())
    o.softmax_attend = f


def m_rope_sign(o):
    def f(x, pos, base=10000.0):
        ang = o.rope_angles(pos, x.shape[-1], base)
        c, s = np.cos(ang), np.sin(ang)
        out = np.empty_like(x, dtype=np.float64)
        out[0::2] = x[0::2] * c + x[1::2] * s
        out[1::2] = -x[0::2] * s + x[1::2] * c
        return out
    o.rope_rotate = f


def m_rope_half_split(o):
    def f(x, pos, base=10000.0):
        d = x.shape[-1]
        ang = o.rope_angles(pos, d, base)
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[: d // 2], x[d // 2:]
        return np.concatenate([a * c - b * s, a * s + b * c])
    o.rope_rotate = f


def m_rope_freq(o):
    o.rope_angles = lambda pos, d, base=10000.0: float(pos) * base ** (-np.arange(d // 2) / d)


def m_paged_slot(o):
    o.paged_row = lambda table, b, t, bs: int(table[b][t // bs]) * bs + (t % bs) + (1 if t % bs else 0)


def m_paged_block(o):
    o.paged_row = lambda table, b, t, bs: int(table[b][t // bs]) + (t % bs)


def m_causal_mask(o):
    def f(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
        K = C @ w_uk_h.T
        V = C @ w_uv_h
        S = scale * (q_nope @ K.T + q_pe @ R.T)
        T = S.shape[0]
        S = np.where(np.triu(np.ones((T, T), bool), k=2), -np.inf, S)
        E = np.exp(S - S.max(1, keepdims=True))
        return (E / E.sum(1, keepdims=True)) @ V
    o.causal_prefill = f


def m_chunk_offset(o):
    # the chunk's queries placed at positions 0 .. T-1 instead of n-T .. n-1
    orig = o.chunked_prefill

    def f(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
        T = q_nope.shape[0]
        return orig(q_nope, q_pe, w_uk_h, w_uv_h, C[:T], R[:T], scale)
    o.chunked_prefill = f


def m_chunk_mask_excludes_self(o):
    def f(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
        T, n = q_nope.shape[0], C.shape[0]
        S = scale * (q_nope @ (C @ w_uk_h.T).T + q_pe @ R.T)
        pos = (n - T) + np.arange(T)
        S = np.where(np.arange(n)[None, :] >= pos[:, None], -np.inf, S)
        S[0, 0] = 0.0 if n - T == 0 else S[0, 0]
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        return (E / E.sum(1, keepdims=True)) @ (C @ w_uv_h), (m + np.log(E.sum(1, keepdims=True)))[:, 0]
    o.chunked_prefill = f


def m_fused_query_transposed(o):
    o.fuse_query_weight = lambda w_q_h, w_uk_h: (w_q_h.T @ w_uk_h).T if w_q_h.shape == w_uk_h.shape \
        else w_uk_h.T @ w_q_h[::-1]


def m_fused_output_order(o):
    o.fuse_output_weight = lambda w_uv_h, w_o_h: (w_o_h.T @ w_uv_h.T).T[::-1]


def m_io_output_one_head(o):
    def f(x, q_pe, w_q, w_uk, w_uv, w_o, C, R, scale):
        q_nope = w_q[0] @ x
        out, l = o.decode_head_nonabsorbed(q_nope, q_pe[0], w_uk[0], w_uv[0], C, R, scale)
        return out @ w_o[0], np.full(w_q.shape[0], l)
    o.decode_model_io = f


def m_absorbed_missing_uv(o):
    def f(q_nope, q_pe, w_uk_h, w_uv_h, C, R, scale):
        q_lat = q_nope @ w_uk_h
        o_lat, lse = o.softmax_attend(scale * (C @ q_lat + R @ q_pe), C)
        return o_lat[: w_uv_h.shape[1]], lse
    o.decode_head_absorbed = f


def m_seq_heads_reversed(o):
    # the absorbed query of head h built with the W_UK of another head
    orig = o.decode_seq_absorbed
    o.decode_seq_absorbed = lambda qn, qp, wuk, wuv, C, R, sc: orig(qn, qp, wuk[::-1], wuv, C, R, sc)


def m_seq_softmax_over_heads(o):
    def f(q_nope, q_pe, w_uk, w_uv, C, R, scale):
        q_lat = np.einsum("hk,hkc->hc", q_nope, w_uk)
        S = scale * (C @ q_lat.T + R @ q_pe.T)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        P = E / E.sum(axis=1, keepdims=True)
        return np.einsum("hc,hcv->hv", P.T @ C, w_uv), np.log(E.sum(axis=0))
    o.decode_seq_absorbed = f


def m_proj_transposed(o):
    o.kv_down_project = lambda h, w_dkv, w_kr: (w_dkv.T @ h, w_kr.T @ h)


def m_proj_last_term_dropped(o):
    o.kv_down_project = lambda h, w_dkv, w_kr: (w_dkv[:, :-1] @ h[:-1], w_kr[:, :-1] @ h[:-1])


def m_proj_key_from_latent_weights(o):
    o.kv_down_project = lambda h, w_dkv, w_kr: (w_dkv @ h, w_dkv[-w_kr.shape[0]:] @ h)


def m_proj_key_not_rotated(o):
    def f(h, w_dkv, w_kr, pos, cache_dtype):
        c, k = o.kv_down_project(h, w_dkv, w_kr)
        lat, _, s, codes = o.append_row(c, k, 0, cache_dtype)
        return lat, o.append_row(c, k, 0, cache_dtype)[1], s, codes
    o.project_append_row = f


MUTATIONS = [m_drop_rope_term, m_wrong_scale, m_head_index, m_uv_for_uk_layout,
             m_unnormalised, m_lse_without_max, m_rope_sign, m_rope_half_split, m_rope_freq,
             m_paged_slot, m_paged_block, m_causal_mask, m_absorbed_missing_uv,
             m_seq_heads_reversed, m_seq_softmax_over_heads, m_chunk_offset,
             m_chunk_mask_excludes_self, m_fused_query_transposed, m_fused_output_order,
             m_io_output_one_head,
             m_proj_transposed, m_proj_last_term_dropped, m_proj_key_from_latent_weights,
             m_proj_key_not_rotated]

PINS = P.ALL_DECODE_PINS + [P.pin_paged_rows, P.pin_rope] + P.PROJECTION_PINS


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_pins_catch_mutation(mutation):
    o = fresh_oracle()
    for pin in PINS:          # the healthy copy passes every pin
        if pin is not P.pin_bruteforce:
            pin(o)
    mutation(o)
    caught = []
    for pin in PINS:
        kw = dict(seeds=(0,), ns=(1, 5)) if pin is P.pin_bruteforce else {}
        try:
            pin(o, **kw)
        except Exception:     # AssertionError, or a shape error from a bad operand
            caught.append(pin.__name__)
    assert caught, f"no pin catches {mutation.__name__}"
