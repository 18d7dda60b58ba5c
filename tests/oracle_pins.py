"""Pins of the CPU oracle: checks against facts the oracle's code does not
produce itself (closed forms, invariants, brute force at high precision,
library format conversions). Each check takes the oracle module so the
mutation tests can run the same checks against deliberately broken copies.

Every check raises AssertionError on failure.
"""

from __future__ import annotations

import math

import mpmath
import numpy as np

mpmath.mp.dps = 50


def _rng(seed):
    return np.random.default_rng(seed)


def tiny_case(seed, n, H=2, d_c=8, d_n=4, d_r=2, d_v=3):
    """Random tiny MLA decode problem in float64 (non-square shapes everywhere
    so that a transposed operand cannot go unnoticed)."""
    r = _rng(seed)
    return dict(
        q_nope=r.standard_normal((1, H, d_n)), q_pe=r.standard_normal((1, H, d_r)),
        w_uk=r.standard_normal((H, d_n, d_c)) / math.sqrt(d_c),
        w_uv=r.standard_normal((H, d_c, d_v)) / math.sqrt(d_c),
        C=r.standard_normal((n, d_c)), R=r.standard_normal((n, d_r)),
        scale=1.0 / math.sqrt(d_n + d_r))


def bruteforce_head(case, h):
    """Decode of one head straight from the definition, in 50-digit mpmath:
    key k_t = [W_UK[h] c_t ; k^R_t], value v_t = c_t W_UV[h], query
    [q_nope ; q_pe], weights exp(scale * q.k_t) normalised over t."""
    mp = mpmath.mp
    C, R = case["C"], case["R"]
    n, d_c = C.shape
    wuk, wuv = case["w_uk"][h], case["w_uv"][h]
    qn, qp = case["q_nope"][0, h], case["q_pe"][0, h]
    d_n, d_v, d_r = wuk.shape[0], wuv.shape[1], R.shape[1]
    sc = mp.mpf(case["scale"])
    scores = []
    values = []
    for t in range(n):
        key = [mp.fsum(mp.mpf(wuk[j, c]) * mp.mpf(C[t, c]) for c in range(d_c)) for j in range(d_n)]
        key += [mp.mpf(R[t, r]) for r in range(d_r)]
        q = [mp.mpf(x) for x in qn] + [mp.mpf(x) for x in qp]
        scores.append(sc * mp.fsum(a * b for a, b in zip(q, key)))
        values.append([mp.fsum(mp.mpf(C[t, c]) * mp.mpf(wuv[c, v]) for c in range(d_c)) for v in range(d_v)])
    w = [mp.exp(s) for s in scores]
    z = mp.fsum(w)
    out = [mp.fsum(w[t] * values[t][v] for t in range(n)) / z for v in range(d_v)]
    return np.array([float(x) for x in out]), float(mp.log(z))


def _decode1(orc, case, absorbed=False):
    return orc.decode(case["q_nope"], case["q_pe"], case["w_uk"], case["w_uv"],
                      [case["C"]], [case["R"]], case["scale"], absorbed=absorbed)


def pin_bruteforce(orc, seeds=(0, 1, 2), ns=(1, 2, 5, 8), tol=1e-13):
    for seed in seeds:
        for n in ns:
            case = tiny_case(seed * 100 + n, n)
            out, lse = _decode1(orc, case)
            for h in range(case["w_uk"].shape[0]):
                ref, ref_lse = bruteforce_head(case, h)
                err = np.max(np.abs(out[0, h] - ref)) / max(np.max(np.abs(ref)), 1e-300)
                assert err <= tol, f"brute force mismatch seed={seed} n={n} h={h}: {err}"
                assert abs(lse[0, h] - ref_lse) <= tol * max(1.0, abs(ref_lse)), "lse mismatch"


def pin_single_row(orc):
    """N = 1: softmax of one score is 1, so o = c_0 W_UV[h] whatever the
    query, and lse equals that single score."""
    case = tiny_case(7, 1)
    out, lse = _decode1(orc, case)
    for h in range(2):
        expect = case["C"][0] @ case["w_uv"][h]
        assert np.allclose(out[0, h], expect, rtol=1e-14, atol=1e-14)
        s0 = case["scale"] * (case["q_nope"][0, h] @ (case["w_uk"][h] @ case["C"][0])
                              + case["q_pe"][0, h] @ case["R"][0])
        assert abs(lse[0, h] - s0) <= 1e-14 * max(1, abs(s0))


def pin_zero_query(orc):
    """q = 0: all scores are 0, attention is uniform: o = mean(C) W_UV[h],
    lse = ln N."""
    case = tiny_case(11, 6)
    case["q_nope"][:] = 0
    case["q_pe"][:] = 0
    out, lse = _decode1(orc, case)
    for h in range(2):
        expect = case["C"].mean(axis=0) @ case["w_uv"][h]
        assert np.allclose(out[0, h], expect, rtol=1e-13, atol=1e-15)
        assert abs(lse[0, h] - math.log(6)) < 1e-14


def pin_rope_shift(orc):
    """All RoPE-key rows equal: the RoPE term adds the same constant to every
    score, so o does not depend on q_pe and lse moves by exactly that constant."""
    case = tiny_case(13, 5)
    case["R"][:] = case["R"][0]
    out1, lse1 = _decode1(orc, case)
    delta = np.array([0.7, -1.3])
    case2 = dict(case)
    case2["q_pe"] = case["q_pe"] + delta
    out2, lse2 = _decode1(orc, case2)
    assert np.allclose(out1, out2, rtol=1e-13, atol=1e-15)
    shift = case["scale"] * (delta @ case["R"][0])
    assert np.allclose(lse2 - lse1, shift, atol=1e-13)


def pin_permutation(orc):
    """Attention is a sum over rows: permuting the cache rows changes nothing."""
    case = tiny_case(17, 8)
    out1, lse1 = _decode1(orc, case)
    p = _rng(3).permutation(8)
    case2 = dict(case, C=case["C"][p], R=case["R"][p])
    out2, lse2 = _decode1(orc, case2)
    assert np.allclose(out1, out2, rtol=1e-13, atol=1e-15)
    assert np.allclose(lse1, lse2, rtol=1e-14)


def pin_absorption(orc):
    """Q K^T = (Q W_UK^T) c^T: the absorbed and non-absorbed forms agree to
    float64 rounding."""
    for seed in range(3):
        case = tiny_case(seed + 50, 7, H=3, d_c=16, d_n=5, d_r=4, d_v=6)
        o1, l1 = _decode1(orc, case)
        o2, l2 = _decode1(orc, case, absorbed=True)
        assert np.max(np.abs(o1 - o2)) <= 1e-12 * np.max(np.abs(o1))
        assert np.max(np.abs(l1 - l2)) <= 1e-12 * np.max(np.abs(l1))


def pin_seq_absorbed(orc):
    """The all-heads absorbed form equals the per-head non-absorbed
    definition (itself pinned by brute force) to float64 rounding, on cases
    with distinct head weights and non-square widths, including one row and
    an empty sequence."""
    for seed, n in ((60, 7), (61, 1), (62, 33)):
        case = tiny_case(seed, n, H=3, d_c=16, d_n=5, d_r=4, d_v=6)
        ref, ref_lse = _decode1(orc, case)
        out, lse = orc.decode_seq_absorbed(case["q_nope"][0], case["q_pe"][0], case["w_uk"],
                                           case["w_uv"], case["C"], case["R"], case["scale"])
        assert out.shape == ref[0].shape
        assert np.max(np.abs(out - ref[0])) <= 1e-12 * np.max(np.abs(ref[0]))
        assert np.max(np.abs(lse - ref_lse[0])) <= 1e-12 * max(1.0, np.max(np.abs(ref_lse[0])))
    case = tiny_case(63, 0, H=3, d_c=16, d_n=5, d_r=4, d_v=6)
    out, lse = orc.decode_seq_absorbed(case["q_nope"][0], case["q_pe"][0], case["w_uk"],
                                       case["w_uv"], case["C"], case["R"], case["scale"])
    assert np.all(out == 0) and np.all(lse == -math.inf)


def pin_hand_example(orc):
    """Hand-worked case: one head, d_c=2, d_nope=1, d_rope=1, d_v=1,
    W_UK=[[1,0]] (key = first latent coordinate), W_UV=[[0],[1]] (value =
    second coordinate), q_nope=1, q_pe=0, two rows c_0=(0,v0), c_1=(x,v1)
    with x = sqrt(2) ln 3 and scale 1/sqrt(2). Scores are 0 and ln 3, so the
    weights are 1/4 and 3/4: o = (v0 + 3 v1)/4 and lse = ln 4."""
    v0, v1 = 2.0, -6.0
    x = math.sqrt(2.0) * math.log(3.0)
    out, lse = orc.decode(np.array([[[1.0]]]), np.array([[[0.0]]]),
                          np.array([[[1.0, 0.0]]]), np.array([[[0.0], [1.0]]]),
                          [np.array([[0.0, v0], [x, v1]])], [np.array([[5.0], [-2.0]])],
                          1.0 / math.sqrt(2.0))
    assert abs(out[0, 0, 0] - (v0 + 3 * v1) / 4) < 1e-14
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14


def pin_causal_prefill(orc):
    """[KV cache experiment] the decode of the token at step t over a cache of
    t+1 rows equals row t of full causal attention over the whole sequence."""
    T, H, d_c, d_n, d_r, d_v = 6, 2, 8, 4, 2, 3
    r = _rng(5)
    Qn = r.standard_normal((T, H, d_n))
    Qp = r.standard_normal((T, H, d_r))
    Wuk = r.standard_normal((H, d_n, d_c))
    Wuv = r.standard_normal((H, d_c, d_v))
    C = r.standard_normal((T, d_c))
    R = r.standard_normal((T, d_r))
    sc = 1 / math.sqrt(d_n + d_r)
    for h in range(H):
        full = orc.causal_prefill(Qn[:, h], Qp[:, h], Wuk[h], Wuv[h], C, R, sc)
        for t in range(T):
            o, _ = orc.decode(Qn[t:t + 1], Qp[t:t + 1], Wuk, Wuv, [C[:t + 1]], [R[:t + 1]],
                              sc, heads=[h])
            assert np.allclose(o[0, h], full[t], rtol=1e-12, atol=1e-14)
    # and the first row of causal attention is the first value exactly
    full = orc.causal_prefill(Qn[:, 0], Qp[:, 0], Wuk[0], Wuv[0], C, R, sc)
    assert np.allclose(full[0], C[0] @ Wuv[0], rtol=1e-14)


def pin_chunked_prefill(orc):
    """Chunked prefill, query by query: query i of a chunk of T over n rows is
    the decode of the first n - T + i + 1 rows (the definition of causal
    attention; decode itself is pinned by brute force). A chunk covering the
    whole sequence (T = n) is full causal attention."""
    H, d_c, d_n, d_r, d_v = 2, 8, 4, 2, 3
    r = _rng(31)
    Wuk = r.standard_normal((H, d_n, d_c))
    Wuv = r.standard_normal((H, d_c, d_v))
    sc = 1 / math.sqrt(d_n + d_r)
    for n, T in ((9, 4), (7, 7), (5, 1), (3, 5)):
        C = r.standard_normal((n, d_c))
        R = r.standard_normal((n, d_r))
        Qn = r.standard_normal((T, H, d_n))
        Qp = r.standard_normal((T, H, d_r))
        for h in range(H):
            out, lse = orc.chunked_prefill(Qn[:, h], Qp[:, h], Wuk[h], Wuv[h], C, R, sc)
            assert out.shape == (T, d_v) and lse.shape == (T,)
            for i in range(T):
                k = n - T + i + 1
                if k <= 0:        # before position 0: no row is visible
                    assert np.all(out[i] == 0) and lse[i] == -math.inf
                    continue
                o, l = orc.decode(Qn[i:i + 1], Qp[i:i + 1], Wuk, Wuv, [C[:k]], [R[:k]], sc,
                                  heads=[h])
                assert np.allclose(o[0, h], out[i], rtol=1e-12, atol=1e-14), (n, T, h, i)
                assert abs(l[0, h] - lse[i]) <= 1e-12 * max(1.0, abs(lse[i]))
            if T == n:
                full = orc.causal_prefill(Qn[:, h], Qp[:, h], Wuk[h], Wuv[h], C, R, sc)
                assert np.allclose(full, out, rtol=1e-12, atol=1e-14)


def _io_case(seed, n=6, H=3, d_c=8, d_n=4, d_r=2, d_v=3, d_model=5):
    r = _rng(seed)
    return dict(x=r.standard_normal(d_model), q_pe=r.standard_normal((H, d_r)),
                w_q=r.standard_normal((H, d_n, d_model)), w_uk=r.standard_normal((H, d_n, d_c)),
                w_uv=r.standard_normal((H, d_c, d_v)), w_o=r.standard_normal((H, d_v, d_model)),
                C=r.standard_normal((n, d_c)), R=r.standard_normal((n, d_r)),
                scale=1 / math.sqrt(d_n + d_r))


def pin_fused_io(orc):
    """Offline absorption: decoding with the fused weights W_QK[h] =
    W_UK[h]^T W_Q[h] and W_VO[h] = W_UV[h] W_O[h] equals the unfused
    definition to float64 rounding (associativity, the identity the pages
    rest the absorption on); the unfused definition with one head and
    W_O = I reduces to decode (pinned by brute force) with q_nope = W_Q x."""
    for seed in (70, 71, 72):
        c = _io_case(seed)
        y, lse = orc.decode_model_io(c["x"], c["q_pe"], c["w_q"], c["w_uk"], c["w_uv"], c["w_o"],
                                     c["C"], c["R"], c["scale"])
        w_qk = np.stack([orc.fuse_query_weight(c["w_q"][h], c["w_uk"][h]) for h in range(3)])
        w_vo = np.stack([orc.fuse_output_weight(c["w_uv"][h], c["w_o"][h]) for h in range(3)])
        assert w_qk.shape == (3, 8, 5) and w_vo.shape == (3, 8, 5)
        y2, lse2 = orc.decode_model_io_fused(c["x"], c["q_pe"], w_qk, w_vo, c["C"], c["R"],
                                             c["scale"])
        assert np.max(np.abs(y - y2)) <= 1e-12 * np.max(np.abs(y))
        assert np.max(np.abs(lse - lse2)) <= 1e-12 * max(1.0, np.max(np.abs(lse)))
    c = _io_case(73, H=1, d_v=5, d_model=5)
    c["w_o"] = np.eye(5)[None]
    y, lse = orc.decode_model_io(c["x"], c["q_pe"], c["w_q"], c["w_uk"], c["w_uv"], c["w_o"],
                                 c["C"], c["R"], c["scale"])
    o, l = orc.decode((c["w_q"][0] @ c["x"])[None, None], c["q_pe"][None], c["w_uk"], c["w_uv"],
                      [c["C"]], [c["R"]], c["scale"])
    assert np.allclose(y, o[0, 0], rtol=1e-13, atol=1e-14) and abs(lse[0] - l[0, 0]) < 1e-13


def pin_fused_hand_example(orc):
    """Hand-worked fusion with square, non-symmetric 2x2 blocks, so that a
    product in the wrong order or of a transposed operand gives other
    numbers: W_UK = [[1,2],[3,4]] (d_nope x d_c), W_Q = [[0,1],[2,1]]
    (d_nope x d_model): W_UK^T W_Q = [[6,4],[8,6]] (W_Q^T W_UK = [[6,8],[4,6]],
    W_UK W_Q^T = [[2,4],[4,10]]). W_UV = [[1,0],[2,1]], W_O = [[1,1],[0,2]]:
    W_UV W_O = [[1,1],[2,4]] (W_O W_UV = [[3,1],[4,2]])."""
    w_uk = np.array([[1.0, 2.0], [3.0, 4.0]])
    w_q = np.array([[0.0, 1.0], [2.0, 1.0]])
    assert np.array_equal(orc.fuse_query_weight(w_q, w_uk), [[6.0, 4.0], [8.0, 6.0]])
    w_uv = np.array([[1.0, 0.0], [2.0, 1.0]])
    w_o = np.array([[1.0, 1.0], [0.0, 2.0]])
    assert np.array_equal(orc.fuse_output_weight(w_uv, w_o), [[1.0, 1.0], [2.0, 4.0]])
    # a non-square case: fused shapes are [d_c, d_model]
    assert orc.fuse_query_weight(np.ones((4, 7)), np.ones((4, 9))).shape == (9, 7)
    assert orc.fuse_output_weight(np.ones((9, 4)), np.ones((4, 7))).shape == (9, 7)


def pin_lse_combine(orc):
    """Split the rows in two, decode each part, merge with the log-sum-exp
    weights e^{lse_i - lse}: the merge equals the decode over all rows. This
    pins lse (a wrong lse gives wrong weights)."""
    case = tiny_case(23, 8)
    out, lse = _decode1(orc, case)
    a = dict(case, C=case["C"][:3], R=case["R"][:3])
    b = dict(case, C=case["C"][3:], R=case["R"][3:])
    oa, la = _decode1(orc, a)
    ob, lb = _decode1(orc, b)
    L = np.logaddexp(la, lb)
    merged = np.exp(la - L)[..., None] * oa + np.exp(lb - L)[..., None] * ob
    assert np.allclose(merged, out, rtol=1e-13, atol=1e-15)
    assert np.allclose(L, lse, rtol=1e-14)


def pin_empty(orc):
    out, lse = orc.decode(np.ones((1, 1, 2)), np.ones((1, 1, 1)), np.ones((1, 2, 3)),
                          np.ones((1, 3, 2)), [np.zeros((0, 3))], [np.zeros((0, 1))], 1.0)
    assert np.all(out == 0) and lse[0, 0] == -math.inf


def pin_paged_rows(orc):
    """Hand-computed block-table addressing: block size 4, table [[2, 0], [1, 3]]:
    sequence 0 token 5 -> block 0 slot 1 -> row 1; sequence 1 token 2 ->
    block 1 slot 2 -> row 6; sequence 1 token 7 -> block 3 slot 3 -> row 15."""
    table = np.array([[2, 0], [1, 3]])
    assert orc.paged_row(table, 0, 5, 4) == 1
    assert orc.paged_row(table, 0, 0, 4) == 8
    assert orc.paged_row(table, 1, 2, 4) == 6
    assert orc.paged_row(table, 1, 7, 4) == 15
    assert list(orc.gather_rows(1, 3, seq_capacity=10)) == [10, 11, 12]
    assert list(orc.gather_rows(0, 6, block_table=table, block_size=4)) == [8, 9, 10, 11, 0, 1]


def pin_rope(orc):
    """RoPE facts: position 0 is the identity; every pair keeps its norm;
    pair 0 has frequency 1 (rotation by p radians); pair 16 of 64 has
    frequency 10000^-0.5 = 0.01; R(a)R(b) = R(a+b); <R(p)q, R(p')k> depends
    only on p - p'."""
    r = _rng(9)
    x = r.standard_normal(64)
    y = r.standard_normal(64)
    assert np.array_equal(orc.rope_rotate(x, 0), x)
    z = orc.rope_rotate(x, 123)
    assert np.allclose(np.hypot(z[0::2], z[1::2]), np.hypot(x[0::2], x[1::2]), rtol=1e-14)
    e0 = np.zeros(64)
    e0[0] = 1.0
    e0[32] = 1.0
    w = orc.rope_rotate(e0, 3)
    assert np.allclose(w[0:2], [math.cos(3.0), math.sin(3.0)], atol=1e-15)
    assert np.allclose(w[32:34], [math.cos(0.03), math.sin(0.03)], atol=1e-15)
    assert np.allclose(orc.rope_rotate(orc.rope_rotate(x, 17), 40), orc.rope_rotate(x, 57), atol=1e-12)
    d1 = orc.rope_rotate(x, 100) @ orc.rope_rotate(y, 90)
    d2 = orc.rope_rotate(x, 1010) @ orc.rope_rotate(y, 1000)
    assert abs(d1 - d2) < 1e-11


def pin_projection_hand_example(orc):
    """Hand-worked down-projection with square 2x2 weights (so a transposed
    operand still runs and must give other numbers): W_DKV = [[1,2],[3,4]],
    W_KR = [[0,1],[2,0]], h = (1,-1): c = (1-2, 3-4) = (-1,-1) (W^T h would
    be (-2,-2)); k = (-1, 2) (W^T h would be (-2,1)). At position 1 the key
    pair turns by 1 radian: (-cos 1 - 2 sin 1, -sin 1 + 2 cos 1)."""
    w_dkv = np.array([[1.0, 2.0], [3.0, 4.0]])
    w_kr = np.array([[0.0, 1.0], [2.0, 0.0]])
    h = np.array([1.0, -1.0])
    c, k = orc.kv_down_project(h, w_dkv, w_kr)
    assert np.array_equal(c, [-1.0, -1.0]) and np.array_equal(k, [-1.0, 2.0])
    lat, rope, _, _ = orc.project_append_row(h, w_dkv, w_kr, 0, "f32")
    assert np.array_equal(lat, [-1.0, -1.0]) and np.array_equal(rope, [-1.0, 2.0])
    _, rope, _, _ = orc.project_append_row(h, w_dkv, w_kr, 1, "f32")
    want = [-math.cos(1.0) - 2 * math.sin(1.0), -math.sin(1.0) + 2 * math.cos(1.0)]
    assert np.allclose(rope, want, rtol=1e-7, atol=1e-7)


def pin_projection_basis(orc):
    """A basis vector h = e_i selects column i of both weights (first, middle
    and last coordinate, non-square shapes); the projection is linear in h;
    and a latent key decompressed from the projected latent equals the key of
    the pre-multiplied weights (W_UK W_DKV) h ([TN] equations for c_KV and
    K_t, multiplied in the other order)."""
    r = _rng(21)
    d_model, d_c, d_r = 12, 8, 4
    w_dkv = r.standard_normal((d_c, d_model))
    w_kr = r.standard_normal((d_r, d_model))
    for i in (0, 5, d_model - 1):
        e = np.zeros(d_model)
        e[i] = 1.0
        c, k = orc.kv_down_project(e, w_dkv, w_kr)
        assert np.array_equal(c, w_dkv[:, i]) and np.array_equal(k, w_kr[:, i])
    h1, h2 = r.standard_normal(d_model), r.standard_normal(d_model)
    c1, k1 = orc.kv_down_project(h1, w_dkv, w_kr)
    c2, k2 = orc.kv_down_project(h2, w_dkv, w_kr)
    c3, k3 = orc.kv_down_project(2.0 * h1 - 3.0 * h2, w_dkv, w_kr)
    assert np.allclose(c3, 2.0 * c1 - 3.0 * c2, atol=1e-12)
    assert np.allclose(k3, 2.0 * k1 - 3.0 * k2, atol=1e-12)
    w_uk = r.standard_normal((5, d_c))
    assert np.allclose(w_uk @ c1, (w_uk @ w_dkv) @ h1, atol=1e-12)


def pin_projection_append(orc):
    """The appended row of a projected token: at position 0 the bf16 row is
    the nearest bf16 of every projected value (RoPE is the identity there);
    at another position the latent is unchanged and each key pair keeps the
    norm of the projected pair."""
    r = _rng(22)
    d_model = 96
    w_dkv = r.standard_normal((512, d_model)) / math.sqrt(d_model)
    w_kr = r.standard_normal((64, d_model)) / math.sqrt(d_model)
    h = r.standard_normal(d_model)
    c, k = orc.kv_down_project(h, w_dkv, w_kr)
    lat, rope, _, _ = orc.project_append_row(h, w_dkv, w_kr, 0, "bf16")
    assert np.array_equal(lat, orc.round_to_bf16(c)) and np.array_equal(rope, orc.round_to_bf16(k))
    lat, rope, _, _ = orc.project_append_row(h, w_dkv, w_kr, 4321, "f32")
    assert np.array_equal(lat, orc.round_to_f32(c))
    assert np.allclose(np.hypot(rope[0::2], rope[1::2]), np.hypot(k[0::2], k[1::2]), rtol=1e-6)
    assert not np.allclose(rope, k, rtol=1e-3)


PROJECTION_PINS = [pin_projection_hand_example, pin_projection_basis, pin_projection_append]


ALL_DECODE_PINS = [pin_bruteforce, pin_single_row, pin_zero_query, pin_rope_shift,
                   pin_permutation, pin_absorption, pin_seq_absorbed, pin_hand_example,
                   pin_causal_prefill, pin_chunked_prefill, pin_fused_io,
                   pin_fused_hand_example, pin_lse_combine, pin_empty]
