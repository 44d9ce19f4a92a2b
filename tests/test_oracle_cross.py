"""Pins for the fp64 oracle of attention with Sq != Skv (CPU only).

oracle/cross.py is tied to independent routines: the square oracle
(reference.py) when Sq == Skv or on the last rows of a longer sequence, the
decode oracle (decode.py) for causal and full masks, and a pure-Python loop.
ALiBi is tied to a closed form (geometric weights when all scores are zero)
and to the square oracle with one extra dimension; the distance bias to a
one-distance selection (zero queries), the softmax of the bias when all
scores are zero, ALiBi as a table, and a pure-Python loop over a padded
batch; padded batches to the decode oracle's cache lengths and the square
oracle per sequence.
``test_planted_cross_mistakes_are_caught`` plants plausible mistakes and checks
that a pin fails for each.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import cross as cr
from oracle import decode as dec


def randn(rng, *shape):
    return rng.standard_normal(shape)


def pin_square_case():
    """Sq == Skv is the square attention, for every mask kind."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, S, D = 1, 4, 2, 23, 8
    q, k, v = randn(rng, B, Hq, S, D), randn(rng, B, Hkv, S, D), randn(rng, B, Hkv, S, D)
    for kind, w in (("full", 0), ("causal", 0), ("causal_window", 5)):
        got = cr.cross_attention(q, k, v, kind, w)
        ref = oracle.attention(q, k, v, kind, w)
        assert np.max(np.abs(got - ref)) < 1e-12, kind


def pin_chunk_is_last_rows():
    """A chunk of Sq queries against Skv >= Sq keys gives the last Sq rows of the
    square attention of the whole sequence (queries before the chunk arbitrary)."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, Sq, Skv, D = 2, 6, 3, 7, 30, 8
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    qf = np.concatenate([randn(rng, B, Hq, Skv - Sq, D), q], axis=2)
    rows = list(range(Skv - Sq, Skv))
    for kind, w in (("full", 0), ("causal", 0), ("causal_window", 4), ("causal_window", 40)):
        got = cr.cross_attention(q, k, v, kind, w)
        ref = oracle.attention(qf, k, v, kind, w, rows=rows)
        assert np.max(np.abs(got - ref)) < 1e-12, (kind, w)


def pin_matches_decode_oracle():
    """Causal and full masks agree with the decode oracle (queries at the end
    of a cache holding Skv positions)."""
    rng = np.random.default_rng(13)
    B, Hq, Hkv, Sq, Skv, D = 2, 8, 2, 5, 19, 16
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    for kind in ("full", "causal"):
        got = cr.cross_attention(q, k, v, kind, scale=0.3)
        ref = dec.decode_attention(q, k, v, kind, cache_len=[Skv] * B, scale=0.3)
        assert np.max(np.abs(got - ref)) < 1e-13, kind


def pin_fewer_keys_than_queries():
    """Skv < Sq: the first Sq - Skv queries see no key (zeros); the rest are the
    square attention of the last Skv queries."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 1, 9, 4, 8
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    got = cr.cross_attention(q, k, v, "causal")
    assert np.all(got[:, :, :Sq - Skv] == 0.0)
    ref = oracle.attention(q[:, :, Sq - Skv:], k, v, "causal")
    assert np.max(np.abs(got[:, :, Sq - Skv:] - ref)) < 1e-12
    full = cr.cross_attention(q, k, v, "full")          # full: every query sees all keys
    assert np.all(np.abs(full[:, :, 0]) > 0)


def pin_brute_force_loop():
    """Pure-Python loops on a tiny causal-window case."""
    rng = np.random.default_rng(15)
    Sq, Skv, D, w, scale = 3, 7, 3, 3, 0.9
    q, k, v = randn(rng, 1, 1, Sq, D), randn(rng, 1, 1, Skv, D), randn(rng, 1, 1, Skv, D)
    got = cr.cross_attention(q, k, v, "causal_window", w, scale=scale)
    for i in range(Sq):
        p = i + Skv - Sq
        js = [j for j in range(Skv) if p - w < j <= p]
        s = [scale * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) for j in js]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        for d in range(D):
            want = math.fsum(e[n] * v[0, 0, js[n], d] for n in range(len(js))) / math.fsum(e)
            assert abs(got[0, 0, i, d] - want) < 1e-13


def pin_row_selection():
    """Selected rows are the same rows of the whole output."""
    rng = np.random.default_rng(16)
    q, k, v = randn(rng, 1, 2, 9, 4), randn(rng, 1, 1, 13, 4), randn(rng, 1, 1, 13, 4)
    whole = cr.cross_attention(q, k, v, "causal_window", 3)
    part = cr.cross_attention(q, k, v, "causal_window", 3, rows=[8, 0, 4])
    assert np.array_equal(part, whole[:, :, [8, 0, 4]])


def geometric_weights(r, lo, hi, p, two_sided):
    """Closed form of softmax(-m * dist) over keys lo..hi-1 with r = exp(-m):
    weight of key j is r^|p - j| over the geometric sum of the same powers."""
    def gsum(n):  # 1 + r + ... + r^(n-1)
        return (1.0 - r ** n) / (1.0 - r) if n > 0 else 0.0
    if two_sided:  # keys on both sides of p: distances 0..p-lo and 1..hi-1-p
        total = gsum(p - lo + 1) + (gsum(hi - p) - 1.0)
    else:          # keys lo..p only: distances 0..p-lo
        total = gsum(p - lo + 1)
    return {j: r ** abs(p - j) / total for j in range(lo, hi)}


def pin_alibi_closed_form():
    """With q = 0 every scaled score is 0, so the weights are the ALiBi bias
    alone: geometric in the distance with ratio exp(-m_a) per query head.
    v = identity reads the weights out.  Distinct slopes in each group of
    heads, a scale that is not 1, and Sq < Skv (aligned queries)."""
    B, Hq, Hkv, Sq, Skv = 1, 4, 2, 3, 7
    slopes = np.array([0.3, 0.7, 1.1, 0.05])
    q = np.zeros((B, Hq, Sq, Skv))
    k = np.random.default_rng(17).standard_normal((B, Hkv, Skv, Skv))
    v = np.broadcast_to(np.eye(Skv), (B, Hkv, Skv, Skv)).copy()
    for kind, w in (("causal", 0), ("causal_window", 2), ("full", 0)):
        got = cr.cross_attention(q, k, v, kind, w, scale=0.25, alibi_slopes=slopes)
        for a in range(Hq):
            r = math.exp(-slopes[a])
            for i in range(Sq):
                p = i + Skv - Sq
                lo = max(0, p - w + 1) if kind == "causal_window" else 0
                hi = Skv if kind == "full" else p + 1
                want = geometric_weights(r, lo, hi, p, kind == "full")
                for j in range(Skv):
                    assert abs(got[0, a, i, j] - want.get(j, 0.0)) < 1e-14, (kind, a, i, j)


def pin_alibi_as_extra_dimension():
    """On causal and causal-window masks ALiBi equals plain attention with one
    more dimension: query coordinate m_a / scale, key coordinate j (the bias
    -m_a (p - j) is m_a j up to a per-row constant, which softmax ignores).
    Checked against the square oracle on the whole sequence (chunk rows)."""
    rng = np.random.default_rng(18)
    B, Hq, Hkv, Sq, Skv, D, scale = 2, 4, 2, 6, 17, 8, 0.3
    slopes = np.array([0.02, 0.5, 0.9, 0.13])
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    qf = np.concatenate([randn(rng, B, Hq, Skv - Sq, D), q], axis=2)
    rows = list(range(Skv - Sq, Skv))
    kx = np.concatenate([k, np.broadcast_to(np.arange(Skv, dtype=np.float64)[None, None, :, None],
                                            (B, Hkv, Skv, 1))], axis=3)
    for kind, w in (("causal", 0), ("causal_window", 5)):
        got = cr.cross_attention(q, k, v, kind, w, scale=scale, alibi_slopes=slopes)
        for a in range(Hq):
            qx = np.concatenate([qf[:, a:a + 1], np.full((B, 1, Skv, 1), slopes[a] / scale)],
                                axis=3)
            h = a // (Hq // Hkv)
            vx = np.concatenate([v[:, h:h + 1], np.zeros((B, 1, Skv, 1))], axis=3)
            ref = oracle.attention(qx, kx[:, h:h + 1], vx, kind, w, scale=scale, rows=rows)
            assert np.max(np.abs(got[:, a:a + 1] - ref[..., :D])) < 1e-12, (kind, a)


def pin_ragged_matches_decode_oracle():
    """Valid key counts per sequence (right padding): the decode oracle with
    the same cache lengths; padded keys and values hold NaN."""
    rng = np.random.default_rng(19)
    B, Hq, Hkv, Sq, Skv, D = 4, 6, 2, 3, 21, 8
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    kv_len = [21, 0, 2, 13]
    for b, L in enumerate(kv_len):
        k[b, :, L:] = np.nan
        v[b, :, L:] = np.nan
    for kind in ("causal", "full"):
        got = cr.cross_attention(q, k, v, kind, scale=0.4, kv_len=kv_len)
        ref = dec.decode_attention(q, k, v, kind, cache_len=kv_len, scale=0.4)
        assert np.all(np.isfinite(got))
        assert np.max(np.abs(got - ref)) < 1e-13, kind


def pin_ragged_queries_are_last_rows():
    """Sequence b with q_len valid query rows and kv_len valid keys: its rows
    are the last q_len rows of the square attention over its kv_len
    positions; padded query rows are zero; padded content never leaks."""
    rng = np.random.default_rng(20)
    B, Hq, Hkv, Sq, Skv, D = 3, 4, 4, 5, 11, 8
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    q_len, kv_len = [5, 2, 0], [11, 6, 4]
    for b in range(B):
        q[b, :, q_len[b]:] = np.nan
        k[b, :, kv_len[b]:] = np.nan
        v[b, :, kv_len[b]:] = np.nan
    for kind, w in (("causal", 0), ("causal_window", 3), ("full", 0)):
        got = cr.cross_attention(q, k, v, kind, w, q_len=q_len, kv_len=kv_len)
        assert np.all(np.isfinite(got))
        for b in range(B):
            nq, nk = q_len[b], kv_len[b]
            assert np.all(got[b, :, nq:] == 0.0)
            if nq == 0:
                continue
            qf = np.concatenate([randn(rng, 1, Hq, nk - nq, D), q[b:b + 1, :, :nq]], axis=2)
            ref = oracle.attention(qf, k[b:b + 1, :, :nk], v[b:b + 1, :, :nk], kind, w,
                                   rows=list(range(nk - nq, nk)))
            assert np.max(np.abs(got[b:b + 1, :, :nq] - ref)) < 1e-12, (kind, b)


def pin_alibi_ragged_brute_force():
    """Pure-Python loops: ALiBi (full mask, two-sided distance) on a padded
    batch with q_len < Sq and kv_len < Skv."""
    rng = np.random.default_rng(21)
    B, Hq, Sq, Skv, D, scale = 2, 2, 4, 6, 3, 0.7
    slopes = [0.4, 1.3]
    q, k, v = randn(rng, B, Hq, Sq, D), randn(rng, B, 1, Skv, D), randn(rng, B, 1, Skv, D)
    q_len, kv_len = [3, 4], [5, 6]
    got = cr.cross_attention(q, k, v, "full", scale=scale, alibi_slopes=slopes, q_len=q_len,
                             kv_len=kv_len)
    for b in range(B):
        for a in range(Hq):
            for i in range(q_len[b]):
                p = i + kv_len[b] - q_len[b]
                sc = [scale * math.fsum(q[b, a, i, d] * k[b, 0, j, d] for d in range(D))
                      - slopes[a] * abs(p - j) for j in range(kv_len[b])]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                for d in range(D):
                    want = math.fsum(e[j] * v[b, 0, j, d] for j in range(kv_len[b])) / math.fsum(e)
                    assert abs(got[b, a, i, d] - want) < 1e-13


def _bias_table(fs, Sq, Skv):
    """Distance-bias table whose row a holds f_a(d) for d = -(Skv - 1) .. Sq - 1."""
    return np.array([[f(t - (Skv - 1)) for t in range(Sq + Skv - 1)] for f in fs])


def pin_dist_bias_selects_distance():
    """Zero queries and a bias of 0 at one distance and -80 elsewhere: row i
    takes the value row at key position p_i + d when that key is visible, and
    the mean of its visible values otherwise (all weights equal)."""
    rng = np.random.default_rng(31)
    D = 3
    for Sq, Skv, kind, d in ((5, 9, "full", 1), (9, 9, "full", 1), (9, 4, "full", -1),
                             (6, 11, "causal", -2), (7, 7, "causal_window", -3)):
        q = np.zeros((1, 1, Sq, D))
        k, v = randn(rng, 1, 1, Skv, D), randn(rng, 1, 1, Skv, D)
        table = _bias_table([lambda x, d=d: 0.0 if x == d else -80.0], Sq, Skv)
        got = cr.cross_attention(q, k, v, kind, 4, scale=0.8, dist_bias=table)
        for i in range(Sq):
            p = i + Skv - Sq
            if kind == "full":
                vis = list(range(Skv))
            elif kind == "causal":
                vis = list(range(0, min(Skv, p + 1)))
            else:
                vis = list(range(max(0, p - 3), min(Skv, p + 1)))
            if not vis:
                assert np.all(got[0, 0, i] == 0.0)
                continue
            want = v[0, 0, p + d] if (p + d) in vis else v[0, 0, vis].mean(axis=0)
            assert np.max(np.abs(got[0, 0, i] - want)) < 1e-12, (Sq, Skv, kind, i)


def pin_dist_bias_zero_scores():
    """With zero scores the weights are the softmax of f_a(j - p_i) over the
    visible keys, whatever the scale (the term is not scaled)."""
    rng = np.random.default_rng(32)
    Sq, Skv, D, G = 4, 7, 2, 2
    fs = [lambda x: 0.3 * x - 0.05 * x * x, lambda x: -0.7 * abs(x + 1) + 0.2 * (x > 2)]
    table = _bias_table(fs, Sq, Skv)
    q = np.zeros((1, G, Sq, D))
    k, v = randn(rng, 1, 1, Skv, D), randn(rng, 1, 1, Skv, D)
    for scale in (1.0, 0.37, -2.0):
        got = cr.cross_attention(q, k, v, "causal", scale=scale, dist_bias=table)
        for a in range(G):
            for i in range(Sq):
                p = i + Skv - Sq
                js = list(range(p + 1))
                e = [math.exp(fs[a](j - p)) for j in js]
                for dd in range(D):
                    want = math.fsum(e[n] * v[0, 0, j, dd] for n, j in enumerate(js)) / math.fsum(e)
                    assert abs(got[0, a, i, dd] - want) < 1e-13, (scale, a, i)


def pin_dist_bias_as_alibi():
    """The table -m_a |d| is ALiBi with slopes m_a (the oracle's ALiBi path,
    pinned above), for every mask, with grouped heads."""
    rng = np.random.default_rng(33)
    B, Hq, Hkv, Sq, Skv, D = 1, 4, 2, 6, 10, 4
    slopes = [0.25, 0.9, 0.05, 1.7]
    q, k, v = randn(rng, B, Hq, Sq, D), randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    table = _bias_table([lambda x, m=m: -m * abs(x) for m in slopes], Sq, Skv)
    for kind, w in (("full", 0), ("causal", 0), ("causal_window", 3)):
        got = cr.cross_attention(q, k, v, kind, w, dist_bias=table)
        ref = cr.cross_attention(q, k, v, kind, w, alibi_slopes=slopes)
        assert np.max(np.abs(got - ref)) < 1e-12, kind


def pin_dist_bias_ragged_brute_force():
    """Pure-Python loops: a distance bias on a padded batch (each sequence
    uses the distances of its own positions), grouped heads."""
    rng = np.random.default_rng(34)
    B, Hq, Sq, Skv, D, scale = 2, 2, 4, 6, 3, 0.6
    fs = [lambda x: math.sin(0.9 * x) + 0.1 * x, lambda x: -0.4 * abs(x) + (0.5 if x == 0 else 0.0)]
    table = _bias_table(fs, Sq, Skv)
    q, k, v = randn(rng, B, Hq, Sq, D), randn(rng, B, 1, Skv, D), randn(rng, B, 1, Skv, D)
    q_len, kv_len = [3, 4], [5, 6]
    for kind in ("full", "causal"):
        got = cr.cross_attention(q, k, v, kind, scale=scale, q_len=q_len, kv_len=kv_len,
                                 dist_bias=table)
        for b in range(B):
            assert np.all(got[b, :, q_len[b]:] == 0.0)
            for a in range(Hq):
                for i in range(q_len[b]):
                    p = i + kv_len[b] - q_len[b]
                    js = [j for j in range(kv_len[b]) if kind == "full" or j <= p]
                    sc = [scale * math.fsum(q[b, a, i, d] * k[b, 0, j, d] for d in range(D))
                          + fs[a](j - p) for j in js]
                    m = max(sc)
                    e = [math.exp(x - m) for x in sc]
                    for d in range(D):
                        want = math.fsum(e[n] * v[b, 0, j, d] for n, j in enumerate(js)) / math.fsum(e)
                        assert abs(got[b, a, i, d] - want) < 1e-13, (kind, b, a, i)


def pin_pair_counts():
    assert cr.cross_visible_pairs(4, 10, "full") == 40
    assert cr.cross_visible_pairs(4, 10, "causal") == 7 + 8 + 9 + 10
    assert cr.cross_visible_pairs(4, 10, "causal_window", 3) == 12
    assert cr.cross_visible_pairs(6, 3, "causal") == 1 + 2 + 3


def pin_local_global_square_and_chunk():
    """local_global: Sq == Skv is the square oracle's local+global mask, and a
    chunk of the last Sq queries gives the square oracle's last Sq rows of the
    whole sequence (a global position inside the chunk and one before it)."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, S, D = 1, 4, 2, 40, 8
    q, k, v = randn(rng, B, Hq, S, D), randn(rng, B, Hkv, S, D), randn(rng, B, Hkv, S, D)
    for w, g in ((3, (0, 17, 33)), (0, (5,)), (6, ())):
        got = cr.cross_attention(q, k, v, "local_global", w, global_idx=g)
        ref = oracle.attention(q, k, v, "local_global", w, g)
        assert np.max(np.abs(got - ref)) < 1e-12, (w, g)
        Sq = 11
        got = cr.cross_attention(q[:, :, S - Sq:], k, v, "local_global", w, global_idx=g)
        ref = oracle.attention(q, k, v, "local_global", w, g, rows=list(range(S - Sq, S)))
        assert np.max(np.abs(got - ref)) < 1e-12, (w, g, Sq)


def pin_local_global_ragged():
    """local_global on a padded batch: each sequence is the square oracle on
    its own positions with the global positions it holds; padded rows are
    zero and padded content (NaN) never leaks, also where a global position
    lies past a sequence's end."""
    rng = np.random.default_rng(23)
    B, Hq, Hkv, Sq, Skv, D, w = 3, 2, 1, 9, 30, 8, 2
    g = (1, 12, 25)
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Skv, D), randn(rng, B, Hkv, Skv, D)
    q_len, kv_len = [9, 4, 6], [30, 14, 6]
    for b in range(B):
        q[b, :, q_len[b]:] = np.nan
        k[b, :, kv_len[b]:] = np.nan
        v[b, :, kv_len[b]:] = np.nan
    got = cr.cross_attention(q, k, v, "local_global", w, q_len=q_len, kv_len=kv_len,
                             global_idx=g)
    assert np.all(np.isfinite(got))
    for b in range(B):
        nq, nk = q_len[b], kv_len[b]
        assert np.all(got[b, :, nq:] == 0.0)
        gb = [x for x in g if x < nk]
        qf = np.concatenate([randn(rng, 1, Hq, nk - nq, D), q[b:b + 1, :, :nq]], axis=2)
        ref = oracle.attention(qf, k[b:b + 1, :, :nk], v[b:b + 1, :, :nk], "local_global", w, gb,
                               rows=list(range(nk - nq, nk)))
        assert np.max(np.abs(got[b:b + 1, :, :nq] - ref)) < 1e-12, b


def pin_local_global_brute_force():
    """Pure-Python loops with the visibility rule written out: |p - j| <= w, or
    p global, or j global."""
    rng = np.random.default_rng(24)
    Hq, Sq, Skv, D, w, scale = 1, 5, 12, 3, 1, 0.9
    g = {2, 7}
    q, k, v = randn(rng, 1, Hq, Sq, D), randn(rng, 1, 1, Skv, D), randn(rng, 1, 1, Skv, D)
    got = cr.cross_attention(q, k, v, "local_global", w, scale=scale, global_idx=sorted(g))
    for i in range(Sq):
        p = i + Skv - Sq
        js = [j for j in range(Skv) if abs(p - j) <= w or p in g or j in g]
        sc = [scale * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) for j in js]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        for d in range(D):
            want = math.fsum(e[t] * v[0, 0, j, d] for t, j in enumerate(js)) / math.fsum(e)
            assert abs(got[0, 0, i, d] - want) < 1e-13
    assert cr.cross_visible_pairs(Sq, Skv, "local_global", w, sorted(g)) == sum(
        len([j for j in range(Skv) if abs(i + Skv - Sq - j) <= w or i + Skv - Sq in g or j in g])
        for i in range(Sq))


PINS = [pin_square_case, pin_chunk_is_last_rows, pin_matches_decode_oracle,
        pin_fewer_keys_than_queries, pin_brute_force_loop, pin_row_selection,
        pin_alibi_closed_form, pin_alibi_as_extra_dimension, pin_ragged_matches_decode_oracle,
        pin_ragged_queries_are_last_rows, pin_alibi_ragged_brute_force, pin_pair_counts,
        pin_local_global_square_and_chunk, pin_local_global_ragged,
        pin_local_global_brute_force, pin_dist_bias_selects_distance, pin_dist_bias_zero_scores,
        pin_dist_bias_as_alibi, pin_dist_bias_ragged_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_cross_pin(pin):
    pin()


_ORIG = cr.cross_visible_range


def _mut_top_left(Sq, Skv, i, kind, window=0):
    # queries aligned with the first keys instead of the last
    return _ORIG(Skv, Skv, i, kind, window)


def _mut_window_wide(Sq, Skv, i, kind, window=0):
    lo, hi = _ORIG(Sq, Skv, i, kind, window)
    return (max(0, lo - 1), hi) if kind == "causal_window" else (lo, hi)


def _mut_full_is_causal(Sq, Skv, i, kind, window=0):
    return _ORIG(Sq, Skv, i, "causal" if kind == "full" else kind, window)


_ORIG_PEN, _ORIG_SLOPE, _ORIG_LENS = cr.alibi_penalty, cr.head_slope, cr.sequence_lengths
_ORIG_DB = cr.distance_bias
_ORIG_KEYS = cr.cross_visible_keys


def _lg_variant(global_query_by_index=False, global_keys=True, one_sided=False, keep_past_end=False):
    """cross_visible_keys with one step of the local_global rule changed."""
    def f(Sq, Skv, i, kind, window=0, global_idx=()):
        if kind != "local_global":
            return _ORIG_KEYS(Sq, Skv, i, kind, window, global_idx)
        p = i + Skv - Sq
        g = sorted({int(x) for x in global_idx if keep_past_end or int(x) < Skv})
        if (i if global_query_by_index else p) in g:
            return np.arange(Skv, dtype=np.int64)
        band = set(range(max(0, p - window), min(Skv, p + (0 if one_sided else window) + 1)))
        return np.array(sorted(band | (set(g) if global_keys else set())), dtype=np.int64)
    return f

MUTATIONS = {
    "top_left_alignment": ("cross_visible_range", _mut_top_left),
    "window_one_too_wide": ("cross_visible_range", _mut_window_wide),
    "full_mask_is_causal": ("cross_visible_range", _mut_full_is_causal),
    # ALiBi rewards distance instead of penalising it
    "alibi_sign": ("alibi_penalty", lambda m, p, j: -_ORIG_PEN(m, p, j)),
    # signed distance: wrong for keys after the query (full mask)
    "alibi_signed_distance": ("alibi_penalty",
                              lambda m, p, j: m * (p - np.asarray(j, dtype=np.float64))),
    # the bias scaled like the scores
    "alibi_scaled": ("alibi_penalty", lambda m, p, j: 0.5 * _ORIG_PEN(m, p, j)),
    # slope of the key/value head instead of the query head
    "alibi_slope_by_kv_head": ("head_slope", lambda sl, a, G: sl[(a // G) * G]),
    # distance measured from the key to the query
    "dist_bias_sign": ("distance_bias",
                       lambda row, p, j, Skv: np.asarray(row, dtype=np.float64)[
                           p - np.asarray(j, dtype=np.int64) + Skv - 1]),
    # table offset taken from the query count (Sq - 1) instead of Skv - 1
    "dist_bias_offset_by_queries": ("distance_bias",
                                    lambda row, p, j, Skv: np.asarray(row, dtype=np.float64)[
                                        np.asarray(j, dtype=np.int64) - p + len(row) - Skv]),
    # the term scaled like the scores
    "dist_bias_scaled": ("distance_bias", lambda row, p, j, Skv: 0.5 * _ORIG_DB(row, p, j, Skv)),
    # row of the key/value head's first query head
    "dist_bias_row_by_kv_head": ("head_bias_row", lambda t, a, G: t[(a // G) * G]),
    # padding ignored: every key and query row valid
    "padding_ignored": ("sequence_lengths", lambda Sq, Skv, ql, kl, b: (Sq, Skv)),
    "lg_global_query_by_row_index": ("cross_visible_keys", _lg_variant(global_query_by_index=True)),
    "lg_global_keys_ignored": ("cross_visible_keys", _lg_variant(global_keys=False)),
    "lg_band_one_sided": ("cross_visible_keys", _lg_variant(one_sided=True)),
    "lg_globals_past_end_kept": ("cross_visible_keys", _lg_variant(keep_past_end=True)),
    # valid query rows counted, but aligned as if all Sq rows were valid
    "ragged_queries_misaligned": ("sequence_lengths",
                                  lambda Sq, Skv, ql, kl, b: (
                                      _ORIG_LENS(Sq, Skv, ql, kl, b)[0],
                                      _ORIG_LENS(Sq, Skv, ql, kl, b)[1]
                                      + Sq - _ORIG_LENS(Sq, Skv, ql, kl, b)[0])),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_cross_mistakes_are_caught(monkeypatch, mutation):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(cr, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {mutation}"
