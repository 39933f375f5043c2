"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics, not by the
oracle itself.  Each pin takes an oracle object (see oracle.Oracle) and raises
AssertionError when the oracle disagrees.  test_oracle_pins.py runs them against the
real oracle and against deliberately altered builds of it.

Sources: page "GPU 内核与 FlashAttention" section 10 (attention as S = QK^T with a
1/sqrt(d)-type scale, softmax, PV), section 11.1 (safe softmax), sections 11.2-11.3
(the blockwise recurrence is exact), section 13.2 (LSE = m + log l), section 14.2
(grouped K/V heads: several query heads index one K/V head, nothing copied) and
section 14.4 (causal: scores with j > i are -inf; blocks wholly above the diagonal can
be skipped without changing the result), section 13.1 (the backward pass: the gradients
of phi = <dO, O>, which finite differences of the forward oracle must reproduce).
"""
import json
import math
import os

import numpy as np
from scipy.special import logsumexp, softmax

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _one_head(x):
    """[N, D] -> [1, N, 1, D]"""
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(1, x.shape[0], 1, x.shape[1])


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def pin_hand_2x2(orc):
    g = _golden("hand_cases.json")["hand_2x2"]
    o, lse = orc.attention(_one_head(g["q"]), _one_head(g["k"]), _one_head(g["v"]), g["scale"])
    e = math.e
    closed_p = np.array([[e / (1 + e), 1 / (1 + e)], [1 / (1 + e), e / (1 + e)]])
    closed_o = closed_p @ np.array(g["v"], dtype=np.float64)
    np.testing.assert_allclose(o[0, :, 0, :], closed_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, :, 0, :], np.array(g["O"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], [math.log(1 + e)] * 2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], g["LSE"], rtol=0, atol=1e-12)


def pin_hand_4x4(orc):
    g = _golden("hand_cases.json")["hand_4x4"]
    o, lse = orc.attention(_one_head(g["q"]), _one_head(g["k"]), _one_head(g["v"]), g["scale"])
    v = np.array(g["v"], dtype=np.float64)
    for i, s in enumerate([0.5, 1.0, 1.5, 2.0]):
        den = math.exp(s) + 3.0
        p = np.full(4, 1.0 / den)
        p[i] = math.exp(s) / den
        np.testing.assert_allclose(o[0, i, 0, :], p @ v, rtol=0, atol=1e-12)
        assert abs(lse[0, 0, i] - math.log(den)) < 1e-12
    np.testing.assert_allclose(o[0, :, 0, :], np.array(g["O"]), rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse[0, 0], g["LSE"], rtol=0, atol=1e-12)


def pin_values_one(orc):
    """V = 1 everywhere: every output is a convex combination of ones, so O = 1."""
    rng = np.random.default_rng(11)
    q, k = _rand(rng, 2, 33, 3, 16), _rand(rng, 2, 47, 3, 16)
    o, _ = orc.attention(q, k, np.ones_like(k), 0.25)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-12)


def pin_identical_keys(orc):
    """All keys equal: scores are constant along a row, so O_i = mean_j v_j and
    LSE_i = s_i + ln Nk with s_i = scale <q_i, k>."""
    rng = np.random.default_rng(12)
    nk, d = 37, 8
    q = _rand(rng, 1, 5, 2, d)
    k = np.broadcast_to(_rand(rng, 1, 1, 2, d), (1, nk, 2, d)).copy()
    v = _rand(rng, 1, nk, 2, d)
    scale = 0.3
    o, lse = orc.attention(q, k, v, scale)
    for h in range(2):
        mean_v = v[0, :, h, :].mean(axis=0)
        for i in range(5):
            np.testing.assert_allclose(o[0, i, h], mean_v, rtol=0, atol=1e-12)
            s = scale * float(q[0, i, h] @ k[0, 0, h])
            assert abs(lse[0, h, i] - (s + math.log(nk))) < 1e-12


def pin_dominant_logit(orc):
    """One key aligned with the query by a large factor: its weight is all but 1, so
    O_i is that key's value row to within exp(-gap) * max|v|, and LSE_i is its score."""
    rng = np.random.default_rng(13)
    d, nk, jstar = 16, 20, 7
    q = _rand(rng, 1, 1, 1, d)
    k = _rand(rng, 1, nk, 1, d) * 0.1
    k[0, jstar, 0] = 40.0 * q[0, 0, 0]
    v = _rand(rng, 1, nk, 1, d)
    o, lse = orc.attention(q, k, v, 1.0)
    s = (k[0, :, 0] @ q[0, 0, 0])
    gap = s[jstar] - np.max(np.delete(s, jstar))
    assert gap > 40
    bound = nk * math.exp(-gap) * np.abs(v).max() * 2
    np.testing.assert_allclose(o[0, 0, 0], v[0, jstar, 0], rtol=0, atol=max(bound, 1e-12))
    assert abs(lse[0, 0, 0] - s[jstar]) < max(nk * math.exp(-gap), 1e-12)


def pin_value_identity_is_softmax(orc):
    """Nk = d and V = I: row i of O is row i of P = softmax(scale q K^T), compared with
    scipy's softmax and logsumexp on numpy's product (Nq != Nk, asymmetric Q and K)."""
    rng = np.random.default_rng(14)
    d = 24
    q, k = _rand(rng, 1, 9, 1, d), _rand(rng, 1, d, 1, d)
    v = np.eye(d).reshape(1, d, 1, d)
    scale = 0.37
    o, lse = orc.attention(q, k, v, scale)
    s = scale * (q[0, :, 0, :] @ k[0, :, 0, :].T)
    np.testing.assert_allclose(o[0, :, 0, :], softmax(s, axis=1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), rtol=0, atol=1e-12)


def pin_single_key(orc):
    """Nk = 1: the only weight is 1, O_i = v_0 and LSE_i = scale <q_i, k_0>."""
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 2, 6, 2, 8), _rand(rng, 2, 1, 2, 8), _rand(rng, 2, 1, 2, 8)
    o, lse = orc.attention(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, 0.7 * np.einsum("bihd,bhd->bhi", q, k[:, 0]), rtol=0, atol=1e-12)


def pin_permutations_and_linearity(orc):
    """Permuting keys with their values leaves O unchanged; permuting queries permutes
    O's rows; O is linear in V."""
    rng = np.random.default_rng(16)
    q, k, v, v2 = (_rand(rng, 1, 11, 2, 8), _rand(rng, 1, 13, 2, 8), _rand(rng, 1, 13, 2, 8),
                   _rand(rng, 1, 13, 2, 8))
    o, lse = orc.attention(q, k, v, 0.5)
    pk = rng.permutation(13)
    o2, lse2 = orc.attention(q, k[:, pk], v[:, pk], 0.5)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)
    pq = rng.permutation(11)
    o3, lse3 = orc.attention(q[:, pq], k, v, 0.5)
    np.testing.assert_allclose(o3, o[:, pq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse3, lse[:, :, pq], rtol=0, atol=1e-12)
    oa, _ = orc.attention(q, k, v2, 0.5)
    ob, _ = orc.attention(q, k, v + 2.0 * v2, 0.5)
    np.testing.assert_allclose(ob, o + 2.0 * oa, rtol=0, atol=1e-12)


def pin_shift_invariance(orc):
    """Adding the same vector u to every key shifts row i's scores by scale <q_i, u>:
    O is unchanged and LSE moves by exactly that amount."""
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 1, 7, 1, 8), _rand(rng, 1, 19, 1, 8), _rand(rng, 1, 19, 1, 8)
    u = _rand(rng, 8) * 3.0
    o, lse = orc.attention(q, k, v, 0.4)
    o2, lse2 = orc.attention(q, k + u, v, 0.4)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2[0, 0] - lse[0, 0], 0.4 * (q[0, :, 0] @ u), rtol=0, atol=1e-11)


def pin_large_logits(orc):
    """Scores of several hundred (exp overflows fp64 past about 709): the max shift keeps
    every value finite; compare with scipy on numpy's product."""
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 1, 8, 1, 16, std=10.0), _rand(rng, 1, 30, 1, 16, std=10.0), _rand(rng, 1, 30, 1, 16)
    o, lse = orc.attention(q, k, v, 2.0)
    s = 2.0 * (q[0, :, 0] @ k[0, :, 0].T)
    assert np.abs(s).max() > 750
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(o[0, :, 0], softmax(s, axis=1) @ v[0, :, 0], rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), rtol=1e-14, atol=1e-10)


def pin_online_recurrence_is_exact(orc):
    """The blockwise recurrence (two-block merge of (m, l), running output rescaled by
    exp(m - m')) reaches the direct result for any block size."""
    rng = np.random.default_rng(19)
    q, k, v = _rand(rng, 2, 10, 2, 8, std=2.0), _rand(rng, 2, 45, 2, 8, std=2.0), _rand(rng, 2, 45, 2, 8)
    o, lse = orc.attention(q, k, v, 0.6)
    for block in (1, 7, 16, 45, 64):
        ob, lseb = orc.attention_online(q, k, v, 0.6, block)
        np.testing.assert_allclose(ob, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lseb, lse, rtol=0, atol=1e-12)


def pin_varlen_is_per_sequence(orc):
    """Packed sequences attend only within themselves: each sequence's rows equal a
    dense single-sequence call; LSE rows past a sequence's end are left untouched."""
    rng = np.random.default_rng(20)
    lens = [5, 1, 12, 8]
    cu = np.concatenate([[0], np.cumsum(lens)])
    total, h, d = int(cu[-1]), 2, 8
    q, k, v = _rand(rng, total, h, d), _rand(rng, total, h, d), _rand(rng, total, h, d)
    o, lse = orc.attention(q, k, v, 0.45, cu_seqlens=cu, max_seqlen=max(lens))
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        od, lsed = orc.attention(q[None, sl], k[None, sl], v[None, sl], 0.45)
        np.testing.assert_allclose(o[sl], od[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b, :, :L], lsed[0], rtol=0, atol=1e-12)
        assert np.all(np.isnan(lse[b, :, L:]))


def pin_rows_match_full(orc):
    """The selected-rows entry point returns the same rows as the full one."""
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 2, 9, 3, 8), _rand(rng, 2, 14, 3, 8), _rand(rng, 2, 14, 3, 8)
    o, lse = orc.attention(q, k, v, 0.5)
    rows = [(0, 0, 0), (1, 2, 8), (0, 1, 4), (1, 0, 3)]
    orow, lrow = orc.attention_rows(q, k, v, 0.5, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(orow[n], o[b, i, h], rtol=0, atol=1e-14)
        assert abs(lrow[n] - lse[b, h, i]) < 1e-14


def pin_causal_hand_3x3(orc):
    """q = k = I_3, v = [[0,1,2],[3,4,5],[6,7,8]], scale 1, causal.  Row i sees keys 0..i with
    scores delta_ij: row 0 is v_0 with LSE 1; row 1 weighs (v_0, v_1) by (1, e)/(1+e) with
    LSE ln(1+e); row 2 weighs (v_0, v_1, v_2) by (1, 1, e)/(2+e) with LSE ln(2+e)."""
    e = math.e
    eye = np.eye(3)
    v = np.arange(9, dtype=np.float64).reshape(3, 3)
    o, lse = orc.attention(_one_head(eye), _one_head(eye), _one_head(v), 1.0, causal=True)
    want = [v[0], (v[0] + e * v[1]) / (1 + e), (v[0] + v[1] + e * v[2]) / (2 + e)]
    np.testing.assert_allclose(o[0, :, 0, :], np.array(want), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], [1.0, math.log(1 + e), math.log(2 + e)], rtol=0, atol=1e-12)


def pin_causal_identical_keys(orc):
    """All keys equal, causal: row i averages the values of keys 0..min(i, Nk-1) and its LSE
    is s_i + ln(min(i+1, Nk)); rows past Nk (Nq > Nk) see every key."""
    rng = np.random.default_rng(22)
    nq, nk, d = 9, 6, 8
    q = _rand(rng, 1, nq, 2, d)
    k = np.broadcast_to(_rand(rng, 1, 1, 2, d), (1, nk, 2, d)).copy()
    v = _rand(rng, 1, nk, 2, d)
    o, lse = orc.attention(q, k, v, 0.4, causal=True)
    for h in range(2):
        for i in range(nq):
            n = min(i + 1, nk)
            np.testing.assert_allclose(o[0, i, h], v[0, :n, h].mean(axis=0), rtol=0, atol=1e-12)
            s = 0.4 * float(q[0, i, h] @ k[0, 0, h])
            assert abs(lse[0, h, i] - (s + math.log(n))) < 1e-12


def pin_causal_value_identity(orc):
    """Nk = d, V = I, causal: O_i is row i of the masked softmax, exactly 0 past column i,
    and scipy's softmax / logsumexp of the first i+1 scores before it."""
    rng = np.random.default_rng(23)
    d = 12
    q, k = _rand(rng, 1, d, 1, d), _rand(rng, 1, d, 1, d)
    v = np.eye(d).reshape(1, d, 1, d)
    o, lse = orc.attention(q, k, v, 0.5, causal=True)
    s = 0.5 * (q[0, :, 0, :] @ k[0, :, 0, :].T)
    for i in range(d):
        assert np.all(o[0, i, 0, i + 1:] == 0.0)
        np.testing.assert_allclose(o[0, i, 0, :i + 1], softmax(s[i, :i + 1]), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - logsumexp(s[i, :i + 1])) < 1e-12


def pin_causal_is_prefix_attention(orc):
    """Causal row i equals unmasked attention of query i over keys 0..i alone (for Nq < Nk
    and Nq > Nk alike)."""
    rng = np.random.default_rng(24)
    for nq, nk in ((7, 11), (11, 7)):
        q, k, v = _rand(rng, 2, nq, 2, 8), _rand(rng, 2, nk, 2, 8), _rand(rng, 2, nk, 2, 8)
        o, lse = orc.attention(q, k, v, 0.55, causal=True)
        for i in range(nq):
            n = min(i + 1, nk)
            op, lsep = orc.attention(q[:, i:i + 1], k[:, :n], v[:, :n], 0.55)
            np.testing.assert_allclose(o[:, i:i + 1], op, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[:, :, i:i + 1], lsep, rtol=0, atol=1e-12)


def pin_causal_block_skipping_is_exact(orc):
    """The blockwise recurrence that skips key blocks lying wholly above the diagonal and
    masks inside the diagonal ones gives the masked definition's result, any block size."""
    rng = np.random.default_rng(25)
    q, k, v = _rand(rng, 1, 20, 2, 8, std=2.0), _rand(rng, 1, 20, 2, 8, std=2.0), _rand(rng, 1, 20, 2, 8)
    o, lse = orc.attention(q, k, v, 0.6, causal=True)
    for block in (1, 3, 8, 20, 64):
        ob, lseb = orc.attention_online(q, k, v, 0.6, block, causal=True)
        np.testing.assert_allclose(ob, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lseb, lse, rtol=0, atol=1e-12)


def pin_causal_varlen_is_per_sequence(orc):
    """Packed causal: every sequence's rows equal a dense causal call on that sequence."""
    rng = np.random.default_rng(26)
    lens = [6, 1, 13]
    cu = np.concatenate([[0], np.cumsum(lens)])
    total = int(cu[-1])
    q, k, v = _rand(rng, total, 2, 8), _rand(rng, total, 2, 8), _rand(rng, total, 2, 8)
    o, lse = orc.attention(q, k, v, 0.45, cu_seqlens=cu, causal=True)
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        od, lsed = orc.attention(q[None, sl], k[None, sl], v[None, sl], 0.45, causal=True)
        np.testing.assert_allclose(o[sl], od[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b, :, :L], lsed[0], rtol=0, atol=1e-12)


def pin_grouped_heads_are_repeated_heads(orc):
    """Grouped K/V heads: with Hkv K/V heads, the result equals ordinary attention on K/V
    with head h // (H / Hkv) copied into head h (MQA at Hkv = 1), dense and packed, plain and
    causal; the selected-rows entry point agrees."""
    rng = np.random.default_rng(27)
    heads = 6
    for hkv in (1, 2, 3):
        g = heads // hkv
        q = _rand(rng, 2, 9, heads, 8)
        k, v = _rand(rng, 2, 13, hkv, 8), _rand(rng, 2, 13, hkv, 8)
        krep, vrep = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
        for causal in (False, True):
            o, lse = orc.attention(q, k, v, 0.5, causal=causal)
            o2, lse2 = orc.attention(q, krep, vrep, 0.5, causal=causal)
            np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-14)
    lens = [4, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = _rand(rng, 13, heads, 8)
    k, v = _rand(rng, 13, 2, 8), _rand(rng, 13, 2, 8)
    o, lse = orc.attention(q, k, v, 0.5, cu_seqlens=cu)
    o2, lse2 = orc.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.5, cu_seqlens=cu)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-14, equal_nan=True)


def pin_heads_are_independent(orc):
    """Attention is defined per (batch, head): each head of a many-head call (dense and
    packed, grouped K/V heads, plain and causal) equals a one-head call on that head's
    Q and its K/V head alone."""
    rng = np.random.default_rng(34)
    heads = 7
    for hkv in (7, 1):
        g = heads // hkv
        q = _rand(rng, 2, 10, heads, 8)
        k, v = _rand(rng, 2, 12, hkv, 8), _rand(rng, 2, 12, hkv, 8)
        for causal in (False, True):
            o, lse = orc.attention(q, k, v, 0.5, causal=causal)
            for h in range(heads):
                sl = slice(h // g, h // g + 1)
                oh, lseh = orc.attention(q[:, :, h:h + 1], k[:, :, sl], v[:, :, sl], 0.5, causal=causal)
                np.testing.assert_allclose(o[:, :, h:h + 1], oh, rtol=0, atol=1e-14)
                np.testing.assert_allclose(lse[:, h:h + 1], lseh, rtol=0, atol=1e-14)
    lens = [3, 8]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = _rand(rng, 11, heads, 8), _rand(rng, 11, heads, 8), _rand(rng, 11, heads, 8)
    o, lse = orc.attention(q, k, v, 0.5, cu_seqlens=cu)
    for h in range(heads):
        oh, lseh = orc.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], 0.5, cu_seqlens=cu)
        np.testing.assert_allclose(o[:, h:h + 1], oh, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, h:h + 1], lseh, rtol=0, atol=1e-14, equal_nan=True)


def pin_grouped_heads_rows_entry(orc):
    """The selected-rows entry point agrees with the full one under grouped K/V heads
    (MQA to groups of 2), plain and causal."""
    rng = np.random.default_rng(33)
    heads = 6
    for hkv in (1, 3):
        g = heads // hkv
        q = _rand(rng, 2, 9, heads, 8)
        k, v = _rand(rng, 2, 13, hkv, 8), _rand(rng, 2, 13, hkv, 8)
        for causal in (False, True):
            o, lse = orc.attention(q, k, v, 0.5, causal=causal)
            rows = [(0, heads - 1, 8), (1, 1, 3), (1, g % heads, 0)]
            orow, lrow = orc.attention_rows(q, k, v, 0.5, rows, causal=causal)
            for n, (b, h, i) in enumerate(rows):
                np.testing.assert_allclose(orow[n], o[b, i, h], rtol=0, atol=1e-14)
                assert abs(lrow[n] - lse[b, h, i]) < 1e-14


def _loss(orc, q, k, v, dout, scale, **kw):
    """phi = <dO, O(q, k, v)>: its gradients are what the backward pass returns."""
    o, _ = orc.attention(q, k, v, scale, **kw)
    return float(np.sum(dout * o))


def _fd_check(orc, q, k, v, dout, scale, rng, n_coords=12, **kw):
    """Central differences of phi at random coordinates of q, k and v against the backward
    oracle (step 1e-5: truncation ~1e-10, rounding ~1e-11)."""
    dq, dk, dv = orc.attention_bwd(q, k, v, dout, scale, **kw)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(n_coords):
            idx = tuple(int(rng.integers(n)) for n in x.shape)
            h = 1e-5
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(orc, args["q"], args["k"], args["v"], dout, scale, **kw)
            args[name] = xm
            fm = _loss(orc, args["q"], args["k"], args["v"], dout, scale, **kw)
            fd = (fp - fm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def pin_bwd_finite_differences(orc):
    """The backward oracle's dQ, dK, dV are the gradients of <dO, O>: central differences of
    the (pinned) forward oracle, plain, causal, grouped heads and packed."""
    rng = np.random.default_rng(28)
    q, k, v = _rand(rng, 2, 7, 4, 8), _rand(rng, 2, 9, 4, 8), _rand(rng, 2, 9, 4, 8)
    dout = _rand(rng, 2, 7, 4, 8)
    _fd_check(orc, q, k, v, dout, 0.5, rng)
    _fd_check(orc, q, k, v, dout, 0.5, rng, causal=True)
    kg, vg = _rand(rng, 2, 9, 2, 8), _rand(rng, 2, 9, 2, 8)
    _fd_check(orc, q, kg, vg, dout, 0.5, rng)
    _fd_check(orc, q, kg[:, :, :1].copy(), vg[:, :, :1].copy(), dout, 0.5, rng, causal=True)
    lens = [3, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qp, kp, vp, dp = (_rand(rng, 10, 4, 8), _rand(rng, 10, 2, 8), _rand(rng, 10, 2, 8), _rand(rng, 10, 4, 8))
    _fd_check(orc, qp, kp, vp, dp, 0.5, rng, cu_seqlens=cu, causal=True)


def pin_bwd_tiny_all_coordinates(orc):
    """Every coordinate of a 3-query, 4-key, d 2 causal case by central differences."""
    rng = np.random.default_rng(29)
    q, k, v, dout = _rand(rng, 1, 3, 1, 2), _rand(rng, 1, 4, 1, 2), _rand(rng, 1, 4, 1, 2), _rand(rng, 1, 3, 1, 2)
    for causal in (False, True):
        _fd_check(orc, q, k, v, dout, 0.9, rng, n_coords=40, causal=causal)


def pin_bwd_value_identities(orc):
    """O is linear in V with rows of P summing to 1: sum_j dV_j = sum_i dO_i (per head), and
    <dV, V> = <dO, O>.  Shifting every key by one vector leaves O unchanged, so the rows of dK
    sum to 0 (per head, under the causal mask too)."""
    rng = np.random.default_rng(30)
    q, k, v, dout = _rand(rng, 2, 11, 2, 8), _rand(rng, 2, 13, 2, 8), _rand(rng, 2, 13, 2, 8), _rand(rng, 2, 11, 2, 8)
    for causal in (False, True):
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, 0.4, causal=causal)
        np.testing.assert_allclose(dv.sum(axis=1), dout.sum(axis=1), rtol=0, atol=1e-12)
        o, _ = orc.attention(q, k, v, 0.4, causal=causal)
        assert abs(np.sum(dv * v) - np.sum(dout * o)) < 1e-11
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)


def pin_bwd_identical_keys_and_single_key(orc):
    """All keys equal: P is uniform (1/Nk), so dV_j = mean_i... = (1/Nk) sum_i dO_i for every j
    and dQ = 0 (dS rows sum to 0 and multiply one key).  Nk = 1: P = 1, dS = 0, so dQ = dK = 0
    and dV_0 = sum_i dO_i."""
    rng = np.random.default_rng(31)
    nk, d = 6, 8
    q, dout = _rand(rng, 1, 5, 2, d), _rand(rng, 1, 5, 2, d)
    k = np.broadcast_to(_rand(rng, 1, 1, 2, d), (1, nk, 2, d)).copy()
    v = _rand(rng, 1, nk, 2, d)
    dq, dk, dv = orc.attention_bwd(q, k, v, dout, 0.3)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, np.broadcast_to(dout.sum(axis=1, keepdims=True) / nk, dv.shape), rtol=0, atol=1e-12)
    dq1, dk1, dv1 = orc.attention_bwd(q, k[:, :1], v[:, :1], dout, 0.3)
    np.testing.assert_allclose(dq1, 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk1, 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv1[:, 0], dout.sum(axis=1), rtol=0, atol=1e-12)


def pin_bwd_rows_match_full(orc):
    """The selected-rows backward returns the full backward's rows: dQ of query rows, dK and dV
    of key rows, dense and packed, plain and causal, grouped heads."""
    rng = np.random.default_rng(32)
    q, dout = _rand(rng, 2, 9, 4, 8), _rand(rng, 2, 9, 4, 8)
    k, v = _rand(rng, 2, 11, 2, 8), _rand(rng, 2, 11, 2, 8)
    for causal in (False, True):
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, 0.5, causal=causal)
        qrows = [(0, 0, 0), (1, 3, 8), (0, 2, 4), (1, 1, 3)]
        krows = [(0, 0, 0), (0, 0, 10), (0, 1, 5), (1, 1, 2), (1, 0, 7)]
        gq, gk, gv = orc.attention_bwd_rows(q, k, v, dout, 0.5, qrows, krows, causal=causal)
        for n, (b, h, i) in enumerate(qrows):
            np.testing.assert_allclose(gq[n], dq[b, i, h], rtol=0, atol=1e-13)
        for n, (b, hk, j) in enumerate(krows):
            np.testing.assert_allclose(gk[n], dk[b, j, hk], rtol=0, atol=1e-13)
            np.testing.assert_allclose(gv[n], dv[b, j, hk], rtol=0, atol=1e-13)
    lens = [4, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qp, dp = _rand(rng, 13, 2, 8), _rand(rng, 13, 2, 8)
    kp, vp = _rand(rng, 13, 2, 8), _rand(rng, 13, 2, 8)
    dq, dk, dv = orc.attention_bwd(qp, kp, vp, dp, 0.5, cu_seqlens=cu, causal=True)
    gq, gk, gv = orc.attention_bwd_rows(qp, kp, vp, dp, 0.5, [(1, 1, 8), (0, 0, 3)], [(1, 0, 0), (1, 1, 8)],
                                        cu_seqlens=cu, causal=True)
    np.testing.assert_allclose(gq[0], dq[4 + 8, 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gq[1], dq[3, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gk[0], dk[4, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gv[1], dv[4 + 8, 1], rtol=0, atol=1e-13)


PINS = [pin_hand_2x2, pin_hand_4x4, pin_values_one, pin_identical_keys, pin_dominant_logit,
        pin_value_identity_is_softmax, pin_single_key, pin_permutations_and_linearity,
        pin_shift_invariance, pin_large_logits, pin_online_recurrence_is_exact,
        pin_varlen_is_per_sequence, pin_rows_match_full, pin_causal_hand_3x3,
        pin_causal_identical_keys, pin_causal_value_identity, pin_causal_is_prefix_attention,
        pin_causal_block_skipping_is_exact, pin_causal_varlen_is_per_sequence,
        pin_grouped_heads_are_repeated_heads, pin_heads_are_independent, pin_grouped_heads_rows_entry,
        pin_bwd_finite_differences, pin_bwd_tiny_all_coordinates,
        pin_bwd_value_identities, pin_bwd_identical_keys_and_single_key, pin_bwd_rows_match_full]

# Pins that need only the forward definition (orc.attention): the whole-matrix oracle is
# held to these as well.
FORWARD_PINS = [pin_hand_2x2, pin_hand_4x4, pin_values_one, pin_identical_keys, pin_dominant_logit,
                pin_value_identity_is_softmax, pin_single_key, pin_permutations_and_linearity,
                pin_shift_invariance, pin_large_logits, pin_varlen_is_per_sequence, pin_causal_hand_3x3,
                pin_causal_identical_keys, pin_causal_value_identity, pin_causal_is_prefix_attention,
                pin_causal_varlen_is_per_sequence, pin_grouped_heads_are_repeated_heads,
                pin_heads_are_independent]
