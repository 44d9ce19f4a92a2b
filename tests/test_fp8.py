"""FP8 (E4M3 and E5M2 inputs, D = 64 and 128) forward pass against the FP8 oracle.

GPU cases compare every output element with oracle.fp8_attention (exact
attention on the decoded E4M3 inputs, fp64) within the per-element bound
oracle.fp8_tolerance derives for the method's rounding of P to E4M3 (the denominator
summed from the rounded weights, as the kernel does on the matrix cores), its fp32
scores, exponentials and accumulation, and the bf16 rounding of the output.
With all queries zero every visible weight is exactly 1, so the output is the
mean of the visible value rows and must match to the output's bf16 rounding:
that case checks masks, tiles and the head mapping tightly.  Host-only cases
check the validation.
"""
import numpy as np
import pytest

import oracle
import workloads

attn = pytest.importorskip("transformer_attention_attn_amd")


def fp8_inputs(B, Hq, Hkv, S, seed, zero_q=False, fmt="e4m3", spread=1.0, D=128):
    inp = workloads.make_inputs(B, Hq, Hkv, S, D, "fp8" if fmt == "e4m3" else "fp8_e5m2", seed)
    if spread != 1.0:  # re-encode the same draws scaled (E5M2's range)
        for n in ("q", "k", "v"):
            inp[n + "_codes"] = workloads.e4m3_codes(
                oracle.fp8_decode(inp[n + "_codes"], fmt) * spread,
                "fp8" if fmt == "e4m3" else "fp8_e5m2")
            inp[n] = workloads.codes_to_float(inp[n + "_codes"],
                                              "fp8" if fmt == "e4m3" else "fp8_e5m2")
    if zero_q:
        inp["q_codes"][:] = 0
        inp["q"][:] = 0.0
    return inp


def run_fp8(device, B, Hq, Hkv, S, mask, window=0, seed=0, scale=None, zero_q=False, rows=None,
            fmt="e4m3", spread=1.0, D=128, global_idx=()):
    import torch

    print(f"fp8 case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {mask} w={window} seed={seed} "
          f"scale={scale} zero_q={zero_q} fmt={fmt} spread={spread} globals={list(global_idx)}",
          flush=True)
    inp = fp8_inputs(B, Hq, Hkv, S, seed, zero_q, fmt, spread, D)
    q, k, v = workloads.to_torch(inp, "fp8" if fmt == "e4m3" else "fp8_e5m2", device)
    o = attn.fwd(q, k, v, mask=mask, window=window, scale=scale,
                 global_idx=list(global_idx) or None)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    got = o.float().cpu().numpy().astype(np.float64)
    codes = (inp["q_codes"], inp["k_codes"], inp["v_codes"])
    ref = oracle.fp8_attention(*codes, mask, window, scale=scale, rows=rows, fmt=fmt,
                               global_idx=global_idx)
    if rows is not None:
        got = got[:, :, rows]
    assert np.all(np.isfinite(got))
    tol = oracle.fp8_tolerance(*codes, mask, window, scale=scale, rows=rows, exact_weights=zero_q,
                               rounded_denominator=True, fmt=fmt, global_idx=global_idx)
    return got, ref, tol


def check(got, ref, tol):
    """Every element within its tolerance (an element whose tolerance is 0,
    e.g. a row whose visible values are exact zeros, must be exact); returns
    the worst error / tolerance ratio."""
    err = np.abs(got - ref)
    assert np.all(err <= tol), float(np.max(err - tol))
    return float(np.max(np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), 0.0)))


SWEEP = []
_rng = np.random.default_rng(94)
for S in (1, 64, 127, 128, 129, 300, 1000, 2049):
    for mask in ("full", "causal", "causal_window"):
        Hq, Hkv = [(8, 2), (4, 4), (8, 1), (16, 2)][int(_rng.integers(4))]
        window = int(_rng.choice([1, 100, 300])) if mask == "causal_window" else 0
        SWEEP.append((1 + int(_rng.integers(2)), Hq, Hkv, S, mask, window))


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"S{c[3]}-{c[4]}-H{c[1]}x{c[2]}")
def test_fp8_sweep(device, case):
    B, Hq, Hkv, S, mask, window = case
    worst = check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + Hq))
    print(f"worst error / tolerance {worst:.3f}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP[::2], ids=lambda c: f"S{c[3]}-{c[4]}-H{c[1]}x{c[2]}")
def test_fp8_zero_queries_exact_means(device, case):
    B, Hq, Hkv, S, mask, window = case
    check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + 7, zero_q=True))


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_fp8_scales(device, scale):
    check(*run_fp8(device, 1, 8, 2, 700, "causal", seed=5, scale=scale))


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"S{c[3]}-{c[4]}-H{c[1]}x{c[2]}")
def test_fp8_d64_sweep(device, case):
    """Head dimension 64 (half the matrix instructions per tile; the LDS rows
    keep their 128-byte layout), E4M3 inputs, the same shapes."""
    B, Hq, Hkv, S, mask, window = case
    worst = check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + Hq + 2, D=64))
    print(f"worst error / tolerance {worst:.3f}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP[::3], ids=lambda c: f"S{c[3]}-{c[4]}-H{c[1]}x{c[2]}")
def test_fp8_d64_zero_queries_and_e5m2(device, case):
    B, Hq, Hkv, S, mask, window = case
    check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + 9, zero_q=True, D=64))
    check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + 10, fmt="e5m2", D=64))
    check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + 11, zero_q=True, fmt="e5m2",
                   D=64))


LG_SWEEP = []
_rng = np.random.default_rng(95)
for D in (64, 128):
    for S in (64, 129, 300, 1000, 2049):
        Hq, Hkv = [(8, 2), (4, 4), (16, 2), (12, 12)][int(_rng.integers(4))]
        window = int(_rng.choice([0, 16, 100, 600]))
        n_g = int(_rng.choice([1, 3, 8, 64]))
        g = sorted({int(x) for x in _rng.integers(0, S, size=n_g)} | ({0} if _rng.integers(2) else set())
                   | ({S - 1} if _rng.integers(2) else set()))[:64]
        LG_SWEEP.append((1 + int(_rng.integers(2)), Hq, Hkv, S, D, window, tuple(g)))


@pytest.mark.gpu
@pytest.mark.parametrize("case", LG_SWEEP, ids=lambda c: f"D{c[4]}-S{c[3]}-w{c[5]}-g{len(c[6])}-H{c[1]}x{c[2]}")
def test_fp8_local_global_sweep(device, case):
    """Local + global tokens: the band, the strip of global keys outside it,
    and the global rows (keys shared out over the waves of a head and merged),
    up to 64 globals, windows 0 to 600."""
    B, Hq, Hkv, S, D, window, g = case
    worst = check(*run_fp8(device, B, Hq, Hkv, S, "local_global", window, seed=S + D + window,
                           D=D, global_idx=g))
    print(f"worst error / tolerance {worst:.3f}")


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_local_global_exact_means_and_e5m2(device, D):
    """Zero queries (each output the mean of its visible values: the band, the
    strip and the global rows tightly) and E5M2 inputs, with globals at both
    ends, next to each other and inside the band."""
    g = (0, 1, 2, 90, 500, 699)
    for window in (0, 5, 1000):
        check(*run_fp8(device, 2, 8, 2, 700, "local_global", window, seed=60 + window, D=D,
                       zero_q=True, global_idx=g))
    check(*run_fp8(device, 1, 12, 12, 700, "local_global", 50, seed=61, D=D, fmt="e5m2",
                   global_idx=g))


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"S{c[3]}-{c[4]}-H{c[1]}x{c[2]}")
def test_fp8_e5m2_sweep(device, case):
    """E5M2 inputs (the instruction's operand formats switched for q, k and
    v; the weights stay E4M3) over the same shapes."""
    B, Hq, Hkv, S, mask, window = case
    worst = check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + Hq + 1, fmt="e5m2"))
    print(f"worst error / tolerance {worst:.3f}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP[1::3], ids=lambda c: f"S{c[3]}-{c[4]}-H{c[1]}x{c[2]}")
def test_fp8_e5m2_zero_queries_exact_means(device, case):
    B, Hq, Hkv, S, mask, window = case
    check(*run_fp8(device, B, Hq, Hkv, S, mask, window, seed=S + 8, zero_q=True, fmt="e5m2"))


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [0.0, -0.002, 0.01])
def test_fp8_e5m2_wide_range(device, scale):
    """Inputs 300 times wider than the others (most beyond E4M3's 448, up to
    about 1500), which only E5M2 holds; small and negative scales keep the
    scores finite and the weights spread."""
    check(*run_fp8(device, 1, 8, 2, 700, "causal", seed=6, scale=scale, fmt="e5m2", spread=300.0))


@pytest.mark.gpu
@pytest.mark.parametrize("name", [n for n, w in workloads.WORKLOADS.items() if w.dtype == "fp8"])
def test_fp8_workload_full_size(device, name):
    """The FP8 workloads at full size, sampled rows, in the benchmark's launch
    configuration."""
    from tests.test_parity import sample_rows

    w = workloads.WORKLOADS[name]
    rows = sample_rows(w)
    got, ref, tol = run_fp8(device, w.B, w.Hq, w.Hkv, w.S, w.mask, w.window, seed=w.seed,
                            rows=rows, D=w.D, global_idx=w.global_idx)
    print(f"fp8 full size: worst error / tolerance {check(got, ref, tol):.3f}", flush=True)


# ----------------------------------------------------------------------------
# host-only
# ----------------------------------------------------------------------------

FAKE = 0x100000


def fp8_status(D=128, mask="causal", window=0, g=None, ptrs=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7),
               S=1000):
    q, k, v, o = ptrs
    return attn.status_string(attn.fwd_raw(q, k, v, o, 1, 8, 2, S, D, mask, window, g, 0.1,
                                           attn.DTYPE_FP8, 0))


def test_fp8_validation():
    assert fp8_status(D=96) == "ATTN_ERR_UNSUPPORTED"
    assert fp8_status(ptrs=(FAKE + 8, FAKE * 3, FAKE * 5, FAKE * 7)) == "ATTN_ERR_ALIGN"
    # o (bf16, 2 bytes per element) overlapping the end of q (1 byte per element)
    nq = 8 * 1000 * 128
    assert fp8_status(ptrs=(FAKE, FAKE * 3, FAKE * 5, FAKE + nq - 16)) == "ATTN_ERR_ALIAS"
    info = attn.plan(1, 32, 8, 8192, 128, "causal", dtype="fp8")
    assert info["kernel"] == 2 and info["keys_per_tile"] == 128
    info = attn.plan(1, 32, 8, 8192, 128, "causal", dtype="fp8_e5m2")
    assert info["kernel"] == 2 and info["keys_per_tile"] == 128
    info = attn.plan(1, 12, 12, 8192, 64, "causal", dtype="fp8")
    assert info["kernel"] == 2 and info["keys_per_tile"] == 128
    assert info["tile_visits"] == 12 * sum(2 * b + 2 for b in range(32))  # 256 rows, 128-key tiles
    assert attn.status_string(attn.fwd_raw(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, 1, 8, 2, 1000, 64,
                                           "local_global", -1, [0], 0.1, attn.DTYPE_FP8_E5M2,
                                           0)) == "ATTN_ERR_WINDOW"
    assert attn.status_string(attn.fwd_raw(FAKE, FAKE * 3, FAKE * 5, FAKE * 7, 1, 8, 2, 1000, 128,
                                           "causal", 0, None, 0.1, 4, 0)) == "ATTN_ERR_UNSUPPORTED"
