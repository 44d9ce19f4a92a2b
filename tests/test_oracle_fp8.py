"""Pins for the FP8 oracle (CPU only).

e4m3_decode and e5m2_decode are checked against hand-decoded codes and against
torch's own float8_e4m3fn and float8_e5m2 types for all 256 codes; the
simulations below decode their inputs with torch, and run for both formats.  fp8_error_bound is checked against a
simulation of what it bounds: the weights of real rows rounded to E4M3 (by
torch's conversion, round to nearest even) at several reference maxima below
the true one, the output formed with the unrounded denominator (bound b) and
with the denominator summed from the rounded weights (bound b'); each bound
must hold everywhere and must not be vacuous.  Planted mistakes in the bound
(a smaller relative unit, no subnormal term) make the simulation exceed it,
in both forms.

fp8_tolerance (the bound plus the kernel's fp32, matrix-instruction and bf16
roundings) is checked against a simulation of the kernel's whole arithmetic:
scores summed as the FP8 instruction sums (groups of 8 products truncated
toward zero 13 bits below the group's largest product, as measured on the
hardware; the simulation reproduces the measured cases) and rounded to fp32,
fp32 exponentials, weights rounded to E4M3, the numerator as 64-key
instruction sums accumulated in fp32 and a sequential fp32 denominator (or,
for the matrix-core denominator, the rounded weights summed by the
instruction), an fp32 division and a bf16 output (nearest even).  With all queries zero the weights are exact, so the fp32 and bf16
terms alone must cover the simulated error; planting a zero bf16 or fp32 unit
makes the simulation exceed the tolerance.
"""
import math

import numpy as np
import pytest

from oracle import fp8 as f8
from oracle import reference as ref


# the global positions the local_global cases use (rows 0..79 or 0..95)
GLOBALS = {"local_global": (3, 40, 77)}


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


def test_e5m2_decode_by_hand():
    codes = np.array([0x3C, 0x7B, 0x01, 0x03, 0x04, 0xC0, 0x00, 0x80, 0x3D, 0x4E], dtype=np.uint8)
    want = [1.0, 57344.0, 2.0 ** -16, 3 * 2.0 ** -16, 2.0 ** -14, -2.0, 0.0, -0.0, 1.25, 24.0]
    got = f8.e5m2_decode(codes)
    assert list(got) == want
    assert list(f8.e5m2_decode(np.array([0x7C, 0xFC], dtype=np.uint8))) == [np.inf, -np.inf]
    assert np.isnan(f8.e5m2_decode(np.array([0x7D, 0x7E, 0x7F, 0xFF], dtype=np.uint8))).all()


def test_e5m2_decode_matches_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy().astype(np.float64)
    got = f8.e5m2_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(got[ok], t[ok])


def _tdtype(fmt):
    import torch

    return {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]


def torch_decode(codes, fmt):
    """Input values by torch's own FP8 types (independent of the oracle)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(codes)).view(_tdtype(fmt)).float().numpy() \
        .astype(np.float64)


def e4m3_round(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).float().numpy().astype(np.float64)


def random_codes(rng, shape, spread=1.0, fmt="e4m3"):
    import torch

    x = (rng.standard_normal(shape) * spread).astype(np.float32)
    return torch.from_numpy(x).to(_tdtype(fmt)).view(torch.uint8).numpy()


def simulate(q, k, v, kind, window, scale, shift, rounded_den=False, fmt="e4m3"):
    """Output of the FP8 method with P rounded to E4M3 while the reference
    maximum sits `shift` (log2 units) below the row maximum; the denominator
    from the unrounded weights, or from the rounded ones (`rounded_den`);
    inputs in format `fmt`, decoded by torch."""
    qd, kd, vd = (torch_decode(x, fmt) for x in (q, k, v))
    B, Hq, S, D = qd.shape
    Hkv = kd.shape[1]
    out = np.empty((B, Hq, S, D))
    rows = np.arange(S)
    for b in range(B):
        for a in range(Hq):
            h = ref.kv_head(a, Hq, Hkv)
            w = ref.weights(qd[b, a], kd[b, h], rows, kind, window, GLOBALS.get(kind, ()), scale)
            p = w / w.max(axis=1, keepdims=True)           # p_max = 1
            pk = e4m3_round(p * 2.0 ** shift) / 2.0 ** shift
            den = (pk if rounded_den else p).sum(axis=1, keepdims=True)
            out[b, a] = (pk @ vd[b, h]) / den
    return out


def check_bound_holds(spread, rounded_den=False, fmt="e4m3"):
    rng = np.random.default_rng(60)
    B, Hq, Hkv, S, D = 1, 4, 2, 96, 16
    q, k, v = (random_codes(rng, s, sp, fmt) for s, sp in (((B, Hq, S, D), spread),
                                                              ((B, Hkv, S, D), spread),
                                                              ((B, Hkv, S, D), 1.0)))
    worst = 0.0
    for kind, w in (("causal", 0), ("full", 0), ("causal_window", 9), ("local_global", 5)):
        g = GLOBALS.get(kind, ())
        exact = f8.fp8_attention(q, k, v, kind, w, scale=0.5, fmt=fmt, global_idx=g)
        bound = f8.fp8_error_bound(q, k, v, kind, w, scale=0.5, rounded_denominator=rounded_den,
                                   fmt=fmt, global_idx=g)
        assert np.all(np.isfinite(bound))
        for shift in (0.0, 0.37, 3.0, 7.9):
            err = np.abs(simulate(q, k, v, kind, w, 0.5, shift, rounded_den, fmt) - exact)
            assert np.all(err <= bound * (1 + 1e-9) + 1e-12), (kind, shift, float((err - bound).max()))
            worst = max(worst, float((err / bound).max()))
    return worst


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rounded_den", [False, True])
def test_bound_holds_and_is_not_vacuous(rounded_den, fmt):
    pytest.importorskip("torch")
    worst = check_bound_holds(1.0, rounded_den, fmt)
    assert worst > 0.05, worst          # the bound is within 20x of a real error
    check_bound_holds(3.0, rounded_den, fmt)  # peaked rows: many weights in the subnormal range


def test_rounded_denominator_bound_vs_unrounded():
    """b' uses |v_j - O| where b uses |v_j|: on values with a large common
    offset b' is the smaller bound (the offset cancels in a weighted mean)."""
    rng = np.random.default_rng(63)
    q = random_codes(rng, (1, 1, 40, 16))
    k = random_codes(rng, (1, 1, 40, 16))
    v = (f8.e4m3_decode(random_codes(rng, (1, 1, 40, 16))) * 0.1 + 8.0).astype(np.float32)
    import torch

    v = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    b = f8.fp8_error_bound(q, k, v, "causal", scale=0.5)
    b2 = f8.fp8_error_bound(q, k, v, "causal", scale=0.5, rounded_denominator=True)
    assert np.all(b2 < b)


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


@pytest.mark.parametrize("rounded_den", [False, True])
@pytest.mark.parametrize("mutation", ["unit_halved", "no_subnormal_term"])
def test_planted_bound_mistakes_are_caught(monkeypatch, mutation, rounded_den):
    pytest.importorskip("torch")
    if mutation == "unit_halved":
        monkeypatch.setattr(f8, "U_E4M3", 2.0 ** -5)
    else:
        monkeypatch.setattr(f8, "ABS_E4M3", 0.0)
    caught = False
    for spread in (1.0, 3.0):
        try:
            check_bound_holds(spread, rounded_den)
        except AssertionError:
            caught = True
    assert caught, mutation
    assert math.isfinite(f8.U_E4M3)


def bf16_round(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).float().numpy().astype(np.float64)


def mfma_sum(prod):
    """Sum over the last axis as the FP8 matrix instruction does (measured):
    groups of 8 consecutive products, each product truncated toward zero to a
    multiple of 2^(E - 13), E the exponent of its group's largest product;
    the truncated products summed exactly (float64 result)."""
    prod = np.asarray(prod, dtype=np.float64)
    n = prod.shape[-1]
    pad = (-n) % 8
    if pad:
        prod = np.concatenate([prod, np.zeros(prod.shape[:-1] + (pad,))], axis=-1)
    g = prod.reshape(prod.shape[:-1] + (-1, 8))
    gmax = np.abs(g).max(axis=-1, keepdims=True)
    grid = np.exp2(np.floor(np.log2(np.where(gmax > 0, gmax, 1.0))) - 13)
    t = np.sign(g) * np.floor(np.abs(g) / grid) * grid
    return t.sum(axis=(-1, -2))


def simulate_kernel(q, k, v, kind, window, scale, shift, round_p=True, bf16_out=True,
                    rounded_den=False, fmt="e4m3"):
    """The FP8 forward's arithmetic on the decoded inputs: scores as the
    matrix instruction sums them (``mfma_sum``) rounded to float32, exponent
    argument and 2^x in float32, weights against a reference maximum `shift`
    log2 units below the row maximum, P rounded to E4M3 (unless round_p is
    False), the numerator as instruction sums of 64 keys accumulated in
    float32, the denominator summed key by key in float32 from the unrounded
    weights (or, `rounded_den`, as instruction sums of the rounded weights),
    one float32 division, the result rounded to bf16 when bf16_out."""
    qd, kd, vd = (torch_decode(x, fmt) for x in (q, k, v))
    B, Hq, S, D = qd.shape
    Hkv = kd.shape[1]
    c = np.float32(abs(scale) / math.log(2.0))
    sign = 1.0 if scale >= 0 else -1.0
    out = np.empty((B, Hq, S, D))
    vis = ref.visibility(np.arange(S), S, kind, window, GLOBALS.get(kind, ()))
    for b in range(B):
        for a in range(Hq):
            h = ref.kv_head(a, Hq, Hkv)
            s = mfma_sum(sign * qd[b, a][:, None, :] * kd[b, h][None, :, :]).astype(np.float32)
            x = np.where(vis, s * c, np.float32(-np.inf)).astype(np.float32)
            m = x.max(axis=1, keepdims=True) - np.float32(shift)
            p = np.exp2((x - m).astype(np.float32)).astype(np.float32)
            pr = e4m3_round(p).astype(np.float32) if round_p else p
            num = np.zeros((S, D), dtype=np.float32)
            for j0 in range(0, S, 64):
                prod = pr[:, None, j0:j0 + 64].astype(np.float64) * vd[b, h, j0:j0 + 64].T[None]
                num = (num + mfma_sum(prod)).astype(np.float32)
            den = np.zeros((S, 1), dtype=np.float32)
            if rounded_den:  # the rounded weights times ones, 64 keys per instruction
                for j0 in range(0, S, 64):
                    den = (den + mfma_sum(pr[:, j0:j0 + 64].astype(np.float64))[:, None]) \
                        .astype(np.float32)
            else:
                for j in range(S):
                    den = (den + p[:, j:j + 1]).astype(np.float32)
            o = (num / den).astype(np.float32)
            out[b, a] = bf16_round(o) if bf16_out else o
    return out


def check_tolerance(spread, exact_weights=False, bf16_out=True, scale=0.5, rounded_den=False,
                    fmt="e4m3", wide_v=False):
    """`wide_v`: values with log-uniform magnitudes over 2^-14 .. 2^2, so that
    the instruction's truncation of small products is exercised."""
    rng = np.random.default_rng(62)
    B, Hq, Hkv, S, D = 1, 2, 1, 80, 32
    q = np.zeros((B, Hq, S, D), dtype=np.uint8) if exact_weights else \
        random_codes(rng, (B, Hq, S, D), spread, fmt)
    k = random_codes(rng, (B, Hkv, S, D), spread, fmt)
    v = random_codes(rng, (B, Hkv, S, D), 1.0, fmt)
    if wide_v:
        import torch

        x = (rng.choice([-1.0, 1.0], size=(B, Hkv, S, D))
             * np.exp2(rng.uniform(-14, 2, size=(B, Hkv, S, D)))).astype(np.float32)
        v = torch.from_numpy(x).to(_tdtype(fmt)).view(torch.uint8).numpy()
    worst = 0.0
    for kind, w in (("causal", 0), ("full", 0), ("causal_window", 9), ("local_global", 5)):
        g = GLOBALS.get(kind, ())
        exact = f8.fp8_attention(q, k, v, kind, w, scale=scale, fmt=fmt, global_idx=g)
        tol = f8.fp8_tolerance(q, k, v, kind, w, scale=scale, exact_weights=exact_weights,
                               bf16_output=bf16_out, rounded_denominator=rounded_den, fmt=fmt,
                               global_idx=g)
        for shift in ((0.0,) if exact_weights else (0.0, 0.37, 3.0, 7.9)):
            got = simulate_kernel(q, k, v, kind, w, scale, shift, round_p=not exact_weights,
                                  bf16_out=bf16_out, rounded_den=rounded_den, fmt=fmt)
            err = np.abs(got - exact)
            assert np.all(err <= tol), (kind, shift, float((err - tol).max()))
            worst = max(worst, float((err / tol).max()))
    return worst


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rounded_den", [False, True])
def test_tolerance_covers_the_kernel_arithmetic(rounded_den, fmt):
    pytest.importorskip("torch")
    assert check_tolerance(1.0, rounded_den=rounded_den, fmt=fmt) > 0.05
    check_tolerance(3.0, rounded_den=rounded_den, fmt=fmt)
    check_tolerance(1.0, scale=-0.3, rounded_den=rounded_den, fmt=fmt)


@pytest.mark.parametrize("mutation", ["e5m2_read_as_e4m3", "e5m2_bias_16"])
def test_planted_e5m2_mistakes_are_caught(monkeypatch, mutation):
    """The oracle's E5M2 decoding with a wrong format or exponent bias: its
    exact output then leaves the simulation (torch's decoding) outside the
    bound."""
    pytest.importorskip("torch")
    if mutation == "e5m2_read_as_e4m3":
        monkeypatch.setattr(f8, "e5m2_decode", f8.e4m3_decode)
    else:
        orig = f8.e5m2_decode
        monkeypatch.setattr(f8, "e5m2_decode", lambda c: orig(c) * 0.5)
    with pytest.raises(AssertionError):
        check_bound_holds(1.0, True, "e5m2")


@pytest.mark.parametrize("rounded_den", [False, True])
def test_tolerance_with_exact_weights(rounded_den):
    pytest.importorskip("torch")
    # the bf16 output rounding is the dominant part: a real error reaches it
    assert check_tolerance(1.0, exact_weights=True, rounded_den=rounded_den) > 0.2
    # without the output rounding only the fp32 terms remain, and they hold
    check_tolerance(1.0, exact_weights=True, bf16_out=False, rounded_den=rounded_den)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rounded_den", [False, True])
def test_tolerance_covers_the_instruction_truncation(rounded_den, fmt):
    """Values spread over 16 binades: many products fall below their group's
    grid, with exact weights (the truncation of P.V alone beside the fp32
    terms) and with real scores."""
    pytest.importorskip("torch")
    check_tolerance(1.0, exact_weights=True, bf16_out=False, rounded_den=rounded_den, fmt=fmt,
                    wide_v=True)
    check_tolerance(1.0, rounded_den=rounded_den, fmt=fmt, wide_v=True)


def test_mfma_sum_matches_the_measured_cases():
    """The simulation's instruction sum reproduces what the hardware returned
    for hand-made rows (2 + 1.5*2^-12 -> 2 + 2^-12; -2 + 1.5*2^-12 -> -2 +
    2^-12; 16 + 1.5*2^-10 -> 16; 2 and 63 values 1.5*2^-14 -> 2 + 56 of them;
    a small value in another group of 8 is kept exactly)."""
    u = 2.0 ** -12
    assert mfma_sum(np.array([2.0, 1.5 * u])) == 2.0 + u
    assert mfma_sum(np.array([-2.0, 1.5 * u])) == -2.0 + u
    assert mfma_sum(np.array([16.0, 1.5 * 2.0 ** -10])) == 16.0
    row = np.full(64, 1.5 * 2.0 ** -14)
    row[0] = 2.0
    assert mfma_sum(row) == 2.0 + 56 * 1.5 * 2.0 ** -14
    row = np.zeros(64)
    row[0], row[20] = 2.0, 1.5 * 2.0 ** -13
    assert mfma_sum(row) == 2.0 + 1.5 * 2.0 ** -13


@pytest.mark.parametrize("rounded_den", [False, True])
@pytest.mark.parametrize("mutation", ["no_bf16_term", "no_fp32_term", "no_truncation_term"])
def test_planted_tolerance_mistakes_are_caught(monkeypatch, mutation, rounded_den):
    pytest.importorskip("torch")
    if mutation == "no_bf16_term":
        monkeypatch.setattr(f8, "U_BF16", 0.0)
        with pytest.raises(AssertionError):
            check_tolerance(1.0, exact_weights=True, rounded_den=rounded_den)
    elif mutation == "no_fp32_term":
        monkeypatch.setattr(f8, "U_F32", 0.0)
        with pytest.raises(AssertionError):
            check_tolerance(1.0, exact_weights=True, bf16_out=False, rounded_den=rounded_den)
    else:
        monkeypatch.setattr(f8, "MFMA_GRID_BITS", 60)
        with pytest.raises(AssertionError):
            check_tolerance(1.0, exact_weights=True, bf16_out=False, rounded_den=rounded_den,
                            fmt="e5m2", wide_v=True)
