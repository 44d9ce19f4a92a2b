"""Pins for the fp64 decode-attention oracle (CPU only).

The decode oracle (oracle/decode.py) is tied to things other than itself: the
full-sequence oracle's last rows (a separate function, pinned in
test_oracle.py), caches whose padding must never leak, closed forms, the
grouped-head reduction to multi-head attention, and a pure-Python loop.
``test_planted_decode_mistakes_are_caught`` plants plausible mistakes in the
decode oracle and checks that some pin fails for each.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import decode as dec


def randn(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_cache_equivalence():
    """Decoding the last Sq positions of a sequence whose keys and values are
    all in the cache gives the full-sequence attention of those rows."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, S, D = 2, 6, 2, 37, 8
    q, k, v = randn(rng, B, Hq, S, D), randn(rng, B, Hkv, S, D), randn(rng, B, Hkv, S, D)
    for Sq in (1, 3, S):
        for kind in ("causal", "full"):
            rows = list(range(S - Sq, S))
            ref = oracle.attention(q, k, v, kind, rows=rows)
            got = dec.decode_attention(q[:, :, S - Sq:], k, v, kind, cache_len=[S] * B)
            assert np.max(np.abs(got - ref)) < 1e-12, (Sq, kind)


def pin_ragged_padding_ignored():
    """Positions beyond a sequence's cache length never reach the output, even
    when they hold NaN; each sequence equals its own truncated cache."""
    rng = np.random.default_rng(2)
    B, Hq, Hkv, Smax, D, Sq = 3, 4, 2, 12, 8, 2
    lens = [5, 12, 2]
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Smax, D), randn(rng, B, Hkv, Smax, D)
    for b, L in enumerate(lens):
        k[b, :, L:] = np.nan
        v[b, :, L:] = np.nan
    for kind in ("causal", "full"):
        got = dec.decode_attention(q, k, v, kind, cache_len=lens)
        assert np.all(np.isfinite(got))
        for b, L in enumerate(lens):
            one = dec.decode_attention(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], kind)
            assert np.max(np.abs(got[b] - one[0])) < 1e-13
            # and the full-sequence oracle on a sequence whose last Sq queries are q
            qf = np.concatenate([randn(rng, 1, Hq, L - Sq, D), q[b:b + 1]], axis=2)
            ref = oracle.attention(qf, k[b:b + 1, :, :L], v[b:b + 1, :, :L], kind,
                                   rows=list(range(L - Sq, L)))
            assert np.max(np.abs(got[b] - ref[0])) < 1e-12


def pin_scale_zero_is_mean():
    """With scale 0 every visible position has the same weight: the output is
    the mean of the visible value rows (causal: the first L - Sq + i + 1)."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, Smax, D, Sq = 2, 2, 1, 9, 4, 3
    lens = [9, 6]
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Smax, D), randn(rng, B, Hkv, Smax, D)
    got = dec.decode_attention(q, k, v, "causal", cache_len=lens, scale=0.0)
    for b, L in enumerate(lens):
        for a in range(Hq):
            for i in range(Sq):
                n = L - Sq + i + 1
                assert np.max(np.abs(got[b, a, i] - v[b, 0, :n].mean(axis=0))) < 1e-13


def pin_grouped_heads_are_repeated_heads():
    """Grouped-query decode equals multi-head decode on K/V repeated G times
    (query head a reads key/value head floor(a / G))."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, Smax, D, Sq = 1, 6, 2, 10, 8, 2
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Smax, D), randn(rng, B, Hkv, Smax, D)
    G = Hq // Hkv
    got = dec.decode_attention(q, k, v, "causal", cache_len=[7])
    ref = dec.decode_attention(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), "causal",
                               cache_len=[7])
    assert np.max(np.abs(got - ref)) < 1e-14
    # and head 3 (group 1) differs from what key/value head 0 would give
    alt = dec.decode_attention(q[:, 3:4], k[:, 0:1], v[:, 0:1], "causal", cache_len=[7])
    assert np.max(np.abs(got[:, 3:4] - alt)) > 1e-3


def pin_brute_force_loop():
    """Pure-Python loops with math.exp / math.fsum on a tiny case."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Smax, D, Sq = 1, 2, 1, 6, 3, 2
    L, scale = 5, 0.7
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Smax, D), randn(rng, B, Hkv, Smax, D)
    got = dec.decode_attention(q, k, v, "causal", cache_len=[L], scale=scale)
    for a in range(Hq):
        for i in range(Sq):
            pos = L - Sq + i
            s = [scale * math.fsum(q[0, a, i, d] * k[0, 0, j, d] for d in range(D))
                 for j in range(pos + 1)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            for d in range(D):
                want = math.fsum(e[j] * v[0, 0, j, d] for j in range(pos + 1)) / tot
                assert abs(got[0, a, i, d] - want) < 1e-13


def pin_edge_rows():
    """A single cached position gives its value row; queries that see no
    position give zeros; with Sq = 1 the causal and full masks coincide."""
    rng = np.random.default_rng(6)
    q = randn(rng, 1, 2, 1, 4)
    k, v = randn(rng, 1, 1, 3, 4), randn(rng, 1, 1, 3, 4)
    got = dec.decode_attention(q, k, v, "full", cache_len=[1])
    assert np.max(np.abs(got[0, :, 0] - v[0, 0, 0])) < 1e-15
    assert np.all(dec.decode_attention(q, k, v, "causal", cache_len=[0]) == 0.0)
    q4 = randn(rng, 1, 2, 4, 4)
    got = dec.decode_attention(q4, k, v, "causal", cache_len=[2])
    assert np.all(got[0, :, :2] == 0.0)              # positions -2, -1: nothing visible
    assert np.max(np.abs(got[0, :, 2] - v[0, 0, 0])) < 1e-15   # sees position 0 only
    a = dec.decode_attention(q, k, v, "causal", cache_len=[3])
    b = dec.decode_attention(q, k, v, "full", cache_len=[3])
    assert np.array_equal(a, b)


def pin_counts():
    """Visible-pair and byte counts against their closed forms."""
    lens = [7, 0, 12]
    Sq, Hq, Hkv, D = 3, 8, 2, 64
    full = dec.decode_effective_flops(Hq, Sq, D, lens, "full")
    assert full == 4 * D * Hq * Sq * sum(lens)
    causal = dec.decode_effective_flops(Hq, Sq, D, lens, "causal")
    want = sum(max(0, L - Sq + i + 1) for L in lens for i in range(Sq))
    assert causal == 4 * D * Hq * want
    assert dec.decode_cache_bytes(3, Hkv, D, lens, 2) == 2 * Hkv * D * 2 * sum(lens)
    for w in (1, 2, 5, 100):
        win = dec.decode_effective_flops(Hq, Sq, D, lens, "causal_window", window=w)
        want = sum(min(w, max(0, L - Sq + i + 1)) for L in lens for i in range(Sq))
        assert win == 4 * D * Hq * want
        # the union of the rows' windows: the last min(L, w + Sq - 1) positions
        nb = dec.decode_cache_bytes(3, Hkv, D, lens, 2, Sq=Sq, kind="causal_window", window=w)
        assert nb == 2 * Hkv * D * 2 * sum(min(L, w + Sq - 1) for L in lens)


def pin_window_cache_equivalence():
    """Under the sliding window, decoding the last Sq positions equals the
    full-sequence oracle's causal_window mask on those rows, at windows below,
    at and above the cache length."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, S, D = 2, 4, 2, 29, 8
    q, k, v = randn(rng, B, Hq, S, D), randn(rng, B, Hkv, S, D), randn(rng, B, Hkv, S, D)
    for Sq in (1, 4, S):
        for w in (1, 3, 11, S, S + 5):
            rows = list(range(S - Sq, S))
            ref = oracle.attention(q, k, v, "causal_window", window=w, rows=rows)
            got = dec.decode_attention(q[:, :, S - Sq:], k, v, "causal_window",
                                       cache_len=[S] * B, window=w)
            assert np.max(np.abs(got - ref)) < 1e-12, (Sq, w)


def pin_window_reads_only_last_positions():
    """Cache positions before a query's window never reach its output, even
    when they hold NaN: the sequence equals the cache cut to its last
    w + Sq - 1 positions; a window that covers the sequence equals causal."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, Smax, D, Sq, w = 3, 4, 1, 40, 8, 3, 6
    lens = [40, 13, 4]
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Smax, D), randn(rng, B, Hkv, Smax, D)
    clean_k, clean_v = k.copy(), v.copy()
    for b, L in enumerate(lens):
        cut = max(0, L - Sq - w + 1)
        k[b, :, :cut] = np.nan
        v[b, :, :cut] = np.nan
        k[b, :, L:] = np.nan
        v[b, :, L:] = np.nan
    got = dec.decode_attention(q, k, v, "causal_window", cache_len=lens, window=w)
    assert np.all(np.isfinite(got))
    for b, L in enumerate(lens):
        cut = max(0, L - Sq - w + 1)
        tail = dec.decode_attention(q[b:b + 1], clean_k[b:b + 1, :, cut:L],
                                    clean_v[b:b + 1, :, cut:L], "causal_window", window=w)
        assert np.max(np.abs(got[b] - tail[0])) < 1e-13
    wide = dec.decode_attention(q, clean_k, clean_v, "causal_window", cache_len=lens, window=Smax)
    causal = dec.decode_attention(q, clean_k, clean_v, "causal", cache_len=lens)
    assert np.array_equal(wide, causal)


def pin_window_closed_forms():
    """Window of one position: the output is the value row at the query's own
    position; scale 0: the mean of the value rows of p - w + 1 .. p."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, Smax, D, Sq = 2, 2, 1, 15, 4, 3
    lens = [15, 9]
    q = randn(rng, B, Hq, Sq, D)
    k, v = randn(rng, B, Hkv, Smax, D), randn(rng, B, Hkv, Smax, D)
    one = dec.decode_attention(q, k, v, "causal_window", cache_len=lens, window=1)
    w = 4
    mean = dec.decode_attention(q, k, v, "causal_window", cache_len=lens, scale=0.0, window=w)
    for b, L in enumerate(lens):
        for i in range(Sq):
            p = L - Sq + i
            for a in range(Hq):
                assert np.max(np.abs(one[b, a, i] - v[b, 0, p])) < 1e-15
                want = v[b, 0, p - w + 1:p + 1].mean(axis=0)
                assert np.max(np.abs(mean[b, a, i] - want)) < 1e-13


PINS = [pin_cache_equivalence, pin_ragged_padding_ignored, pin_scale_zero_is_mean,
        pin_grouped_heads_are_repeated_heads, pin_brute_force_loop, pin_edge_rows, pin_counts,
        pin_window_cache_equivalence, pin_window_reads_only_last_positions,
        pin_window_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_decode_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

_ORIG_RANGE = dec.decode_visible_range
_ORIG_DECODE = dec.decode_attention


def _mut_causal_excludes_own_position(L, Sq, i, kind, window=0):
    lo, hi = _ORIG_RANGE(L, Sq, i, kind, window)
    return (lo, max(lo, hi - 1)) if kind != "full" else (lo, hi)


def _mut_query_at_index(L, Sq, i, kind, window=0):
    # query i taken at position i instead of L - Sq + i
    return _ORIG_RANGE(L, L, i, kind, window) if L >= Sq else _ORIG_RANGE(L, Sq, i, kind, window)


def _mut_window_one_too_wide(L, Sq, i, kind, window=0):
    lo, hi = _ORIG_RANGE(L, Sq, i, kind, window)
    return (max(0, lo - 1), hi) if kind == "causal_window" else (lo, hi)


def _mut_window_from_sequence_start(L, Sq, i, kind, window=0):
    # the window taken as the first w positions rather than the last
    lo, hi = _ORIG_RANGE(L, Sq, i, kind, window)
    return (0, min(hi, window)) if kind == "causal_window" else (lo, hi)


def _mut_window_ignored(L, Sq, i, kind, window=0):
    return _ORIG_RANGE(L, Sq, i, "causal" if kind == "causal_window" else kind, window)


def _mut_ignores_length(q, k_cache, v_cache, kind, cache_len=None, scale=None, window=0):
    return _ORIG_DECODE(q, k_cache, v_cache, kind, cache_len=None, scale=scale, window=window)


def _variant(head=None, normalise=True, use_scale=True):
    """A copy of decode_attention with one step changed."""
    def f(q, k_cache, v_cache, kind, cache_len=None, scale=None, window=0):
        q = np.asarray(q)
        kc, vc = np.asarray(k_cache), np.asarray(v_cache)
        B, Hq, Sq, D = q.shape
        Hkv, Smax = kc.shape[1], kc.shape[2]
        G = Hq // Hkv
        lens = [Smax] * B if cache_len is None else [int(x) for x in cache_len]
        sc = (1.0 / np.sqrt(D) if scale is None else scale) if use_scale else 1.0
        out = np.zeros((B, Hq, Sq, D))
        for b in range(B):
            for a in range(Hq):
                h = a // G if head is None else head(a, Hq, Hkv)
                for i in range(Sq):
                    lo, hi = dec.decode_visible_range(lens[b], Sq, i, kind, window)
                    if hi == lo:
                        continue
                    s = sc * (kc[b, h, lo:hi] @ q[b, a, i])
                    e = np.exp(s - s.max())
                    out[b, a, i] = ((e / e.sum()) if normalise else e) @ vc[b, h, lo:hi]
        return out
    return f


MUTATIONS = {
    "causal_excludes_own_position": ("decode_visible_range", _mut_causal_excludes_own_position),
    "query_at_index_not_cache_end": ("decode_visible_range", _mut_query_at_index),
    "window_one_too_wide": ("decode_visible_range", _mut_window_one_too_wide),
    "window_from_sequence_start": ("decode_visible_range", _mut_window_from_sequence_start),
    "window_ignored": ("decode_visible_range", _mut_window_ignored),
    "cache_length_ignored": ("decode_attention", _mut_ignores_length),
    "head_map_modulo": ("decode_attention", _variant(head=lambda a, Hq, Hkv: a % Hkv)),
    "not_normalised": ("decode_attention", _variant(normalise=False)),
    "scale_ignored": ("decode_attention", _variant(use_scale=False)),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_decode_mistakes_are_caught(monkeypatch, mutation):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(dec, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {mutation}"
