"""Pins for the fp64 oracle of attention with Sq != Skv (CPU only).

oracle/cross.py is tied to independent routines: the square oracle
(reference.py) when Sq == Skv or on the last rows of a longer sequence, the
decode oracle (decode.py) for causal and full masks, and a pure-Python loop.
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


def pin_pair_counts():
    assert cr.cross_visible_pairs(4, 10, "full") == 40
    assert cr.cross_visible_pairs(4, 10, "causal") == 7 + 8 + 9 + 10
    assert cr.cross_visible_pairs(4, 10, "causal_window", 3) == 12
    assert cr.cross_visible_pairs(6, 3, "causal") == 1 + 2 + 3


PINS = [pin_square_case, pin_chunk_is_last_rows, pin_matches_decode_oracle,
        pin_fewer_keys_than_queries, pin_brute_force_loop, pin_row_selection, pin_pair_counts]


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


MUTATIONS = {
    "top_left_alignment": _mut_top_left,
    "window_one_too_wide": _mut_window_wide,
    "full_mask_is_causal": _mut_full_is_causal,
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_cross_mistakes_are_caught(monkeypatch, mutation):
    monkeypatch.setattr(cr, "cross_visible_range", MUTATIONS[mutation])
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {mutation}"
