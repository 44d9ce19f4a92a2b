"""Pins for the FP8 oracle (CPU only).

e4m3_decode is checked against hand-decoded codes and against torch's own
float8_e4m3fn type for all 256 codes.  fp8_error_bound is checked against a
simulation of what it bounds: the weights of real rows rounded to E4M3 (by
torch's conversion, round to nearest even) at several reference maxima below
the true one, the output formed with the unrounded denominator; the bound
must hold everywhere and must not be vacuous.  Planted mistakes in the bound
(a smaller relative unit, no subnormal term) make the simulation exceed it.
"""
import math

import numpy as np
import pytest

from oracle import fp8 as f8
from oracle import reference as ref


def test_e4m3_decode_by_hand():
    codes = np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0xC0, 0x00, 0x80, 0x39, 0x58], dtype=np.uint8)
    want = [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9, -2.0, 0.0, -0.0, 1.125, 16.0]
    got = f8.e4m3_decode(codes)
    assert list(got) == want
    assert np.isnan(f8.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_decode_matches_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = f8.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(got[ok], t[ok])


def e4m3_round(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).float().numpy().astype(np.float64)


def random_codes(rng, shape, spread=1.0):
    import torch

    x = (rng.standard_normal(shape) * spread).astype(np.float32)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def simulate(q, k, v, kind, window, scale, shift):
    """Output of the FP8 method with P rounded to E4M3 while the reference
    maximum sits `shift` (log2 units) below the row maximum."""
    qd, kd, vd = (f8.e4m3_decode(x) for x in (q, k, v))
    B, Hq, S, D = qd.shape
    Hkv = kd.shape[1]
    out = np.empty((B, Hq, S, D))
    rows = np.arange(S)
    for b in range(B):
        for a in range(Hq):
            h = ref.kv_head(a, Hq, Hkv)
            w = ref.weights(qd[b, a], kd[b, h], rows, kind, window, (), scale)
            p = w / w.max(axis=1, keepdims=True)           # p_max = 1
            pk = e4m3_round(p * 2.0 ** shift) / 2.0 ** shift
            out[b, a] = (pk @ vd[b, h]) / p.sum(axis=1, keepdims=True)
    return out


def check_bound_holds(spread):
    rng = np.random.default_rng(60)
    B, Hq, Hkv, S, D = 1, 4, 2, 96, 16
    q, k, v = (random_codes(rng, s, sp) for s, sp in (((B, Hq, S, D), spread),
                                                         ((B, Hkv, S, D), spread),
                                                         ((B, Hkv, S, D), 1.0)))
    worst = 0.0
    for kind, w in (("causal", 0), ("full", 0), ("causal_window", 9)):
        exact = f8.fp8_attention(q, k, v, kind, w, scale=0.5)
        bound = f8.fp8_error_bound(q, k, v, kind, w, scale=0.5)
        for shift in (0.0, 0.37, 3.0, 7.9):
            err = np.abs(simulate(q, k, v, kind, w, 0.5, shift) - exact)
            assert np.all(err <= bound * (1 + 1e-9) + 1e-12), (kind, shift, float((err - bound).max()))
            worst = max(worst, float((err / bound).max()))
    return worst


def test_bound_holds_and_is_not_vacuous():
    pytest.importorskip("torch")
    worst = check_bound_holds(1.0)
    assert worst > 0.05, worst          # the bound is within 20x of a real error
    check_bound_holds(3.0)              # peaked rows: many weights in the subnormal range


def test_zero_queries_give_the_mean_of_visible_values():
    rng = np.random.default_rng(61)
    q = np.zeros((1, 2, 20, 8), dtype=np.uint8)
    k = random_codes(rng, (1, 1, 20, 8))
    v = random_codes(rng, (1, 1, 20, 8))
    vd = f8.e4m3_decode(v)
    got = f8.fp8_attention(q, k, v, "causal_window", 5)
    for i in range(20):
        lo = max(0, i - 4)
        want = vd[0, 0, lo:i + 1].mean(axis=0)
        assert np.max(np.abs(got[0, :, i] - want)) < 1e-12


@pytest.mark.parametrize("mutation", ["unit_halved", "no_subnormal_term"])
def test_planted_bound_mistakes_are_caught(monkeypatch, mutation):
    pytest.importorskip("torch")
    if mutation == "unit_halved":
        monkeypatch.setattr(f8, "U_E4M3", 2.0 ** -5)
    else:
        monkeypatch.setattr(f8, "ABS_E4M3", 0.0)
    caught = False
    for spread in (1.0, 3.0):
        try:
            check_bound_holds(spread)
        except AssertionError:
            caught = True
    assert caught, mutation
    assert math.isfinite(f8.U_E4M3)
