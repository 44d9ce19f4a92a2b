"""fp64 CPU oracle for the FP8 forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP path.

What it computes: the FP8 variant of the fused attention that "Transformer 演进
与变体", section Flash Attention (the FlashAttention-3 paragraph: FP8 for the
matrix products, softmax and accumulation in BF16/FP32), and "第 8 章 AI 算法
Transformer大模型", section 8.6.5 (low precision: kernels with an FP8 forward
pass, per-tensor scale factors) describe: the two matrix products take FP8
(E4M3) operands while the softmax and the accumulation stay in higher
precision.  Reading: per-tensor scale factors are the caller's (folded into
the score scale for q and k, applied to the output for v), so the codes are
taken at face value.

* The inputs q, k, v are E4M3 codes.  ``e4m3_decode`` is the plain definition
  of that format (the OCP 8-bit float: 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits, subnormals below 2^-6, no infinities, 0x7F / 0xFF NaN),
  written from the bit layout.
* Or E5M2 codes (the page names both FP8 formats; ``fmt="e5m2"``):
  ``e5m2_decode`` is that format's plain definition (OCP: 1 sign bit, 5
  exponent bits with bias 15, 2 mantissa bits, subnormals below 2^-14,
  exponent field 31 is infinity with a zero mantissa and NaN otherwise).
  Reading: the weights P are still rounded to E4M3 for the P.V product (the
  weights lie in [0, 1] after the row maximum is taken out, where E4M3's
  extra mantissa bit is the better choice and E5M2's range is not needed),
  so the bound below is the same for both input formats; a product of two
  E5M2 values (3-bit significands) is as exact in fp32 as one of E4M3
  values, so the score terms are unchanged too.
* The reference output is exact masked attention (reference.py) on the decoded
  values: the score product of E4M3 inputs is exact, so the only rounding of
  the method that the oracle does not carry out is the E4M3 rounding of the
  softmax weights P before the P.V product (the second product needs FP8
  operands).

Tolerance, derived from that rounding (reading: P is rounded to nearest,
relative to whatever reference maximum the kernel holds at that moment):
with p_j = exp(s_j - max_i s) of a row's visible keys and L = sum_j p_j,
E4M3 rounding to nearest changes a weight by at most u = 2^-4 of itself in
the normal range and by at most 2^-10 (half the smallest subnormal) below it;
a kernel whose reference maximum is lower than the row's maximum holds the
same weights multiplied by a power of two >= 1, so in units of p_j the error
stays within e_j = u p_j + 2^-10.  With the denominator summed from the
unrounded weights, O - O_exact = sum_j (p~_j - p_j) v_j / L, hence

    |O - O_exact| <= b = sum_j e_j |v_j| / L.

``fp8_error_bound`` returns b per output element.

With the denominator summed from the ROUNDED weights as well (both sums then
run on the matrix cores: P~ times V and P~ times a column of ones), the output
is the exact weighted mean under the rounded weights p~_j, and since
sum_j p_j (v_j - O_exact) = 0,

    O - O_exact = sum_j (p~_j - p_j) (v_j - O_exact) / sum_j p~_j,

with sum_j p~_j >= L - sum_j e_j, hence

    |O - O_exact| <= b' = sum_j e_j |v_j - O_exact| / (L - sum_j e_j)

(no bound when sum_j e_j >= L).  In the normalised weights w_j = p_j / L of
the oracle (w_max = 1 / L, as p_max = 1) e_j / L = u w_j + 2^-10 w_max.
``fp8_error_bound(..., rounded_denominator=True)`` returns b'.

``fp8_tolerance`` adds the kernel's other roundings, each bounded from the
arithmetic it does (first order in the fp32 unit u = 2^-24):

* fp32 scores and exponent.  A score is an fp32 sum of D exact E4M3 products
  (a product of two 4-bit significands fits fp32), error <= D u A_j with
  A_j = sum_d |q_d k_jd|; the exponent argument x = s c - m c (c = |scale|
  log2 e, rounded to fp32) adds at most 4 u c max(A) more, so
  |dx| <= (D + 4) u c max_j A_j, and 2^x with v_exp_f32 (about one ulp) gives
  each weight a relative error of at most ew = ln2 |dx| + 2 u.  Relative
  weight errors of at most ew move a weighted mean by at most 2 ew (1 + 2 ew)
  sum_j p_j |v_j| / L.
* fp32 accumulation.  The numerator sum_j p~_j v_j runs as a chain of fp32
  additions of partial sums of at most 16 keys (n_vis / 16 + 1 steps, plus
  rescales and the final division), error <= (n_vis / 16 + 48) u
  sum_j p_j |v_j| / L; the denominator is a chain of at most n_vis fp32
  additions of positive weights, relative error <= (n_vis + 8) u, which moves
  O by that fraction of |O|; a denominator summed on the matrix cores (the
  rounded weights times ones) is a chain of the numerator's kind, relative
  error <= (n_vis / 16 + 48) u.
* bf16 output.  O is rounded once to bf16 (8-bit significand, nearest even):
  at most 2^-8 of the rounded value, i.e. 2^-8 (|O| + the bounds above).

With all queries zero every weight is exactly 2^0 = 1 (the E4M3 rounding of 1
is exact and the scores are exact zeros), so b and ew vanish and only the
accumulation and output terms remain (``exact_weights=True``).

Pinned by tests/test_oracle_fp8.py.
"""
from __future__ import annotations

import numpy as np

from . import reference

U_E4M3 = 2.0 ** -4          # relative rounding bound in the normal range
ABS_E4M3 = 2.0 ** -10       # absolute rounding bound below it
U_F32 = 2.0 ** -24          # fp32 unit roundoff (24-bit significand)
U_BF16 = 2.0 ** -8          # bf16 unit roundoff (8-bit significand)


def e4m3_decode(codes):
    """Values (float64) of E4M3 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e5m2_decode(codes):
    """Values (float64) of E5M2 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    normal = sign * (1.0 + m / 4.0) * np.exp2(e - 15.0)
    sub = sign * (m / 4.0) * 2.0 ** -14
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 31) & (m == 0), sign * np.inf, val)
    return np.where((e == 31) & (m != 0), np.nan, val)


FP8_FORMATS = ("e4m3", "e5m2")


def fp8_decode(codes, fmt="e4m3"):
    """Values (float64) of FP8 codes in the given input format."""
    if fmt == "e4m3":
        return e4m3_decode(codes)
    if fmt == "e5m2":
        return e5m2_decode(codes)
    raise ValueError(f"unknown FP8 format {fmt!r}")


def fp8_attention(q_codes, k_codes, v_codes, kind, window=0, scale=None, rows=None, fmt="e4m3"):
    """Exact masked attention (float64) on the decoded FP8 inputs."""
    return reference.attention(fp8_decode(q_codes, fmt), fp8_decode(k_codes, fmt),
                               fp8_decode(v_codes, fmt), kind, window, (), scale=scale, rows=rows)


def fp8_error_bound(q_codes, k_codes, v_codes, kind, window=0, scale=None, rows=None,
                    rounded_denominator=False, fmt="e4m3"):
    """Per-element bound (float64, shaped like the output) on the error the
    E4M3 rounding of P can cause: b with the denominator summed from the
    unrounded weights, b' with the denominator summed from the rounded ones
    (``rounded_denominator``; inf where sum_j e_j >= L).  ``fmt``: the input
    format of the codes."""
    q = fp8_decode(q_codes, fmt)
    k = fp8_decode(k_codes, fmt)
    v = fp8_decode(v_codes, fmt)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, Hq, rows.size, D), dtype=np.float64)
    for b in range(B):
        for a in range(Hq):
            h = reference.kv_head(a, Hq, Hkv)
            w = reference.weights(q[b, a, rows], k[b, h], rows, kind, window, (), scale)
            wmax = w.max(axis=1, keepdims=True)
            # w = p / L with p_max = 1, so p = w / wmax and 1 / L = wmax
            e = np.where(w > 0, U_E4M3 * w + ABS_E4M3 * wmax, 0.0)
            if not rounded_denominator:
                out[b, a] = e @ np.abs(v[b, h])
                continue
            o = w @ v[b, h]                                   # O_exact of these rows
            num = np.einsum("rj,rjd->rd", e, np.abs(v[b, h][None, :, :] - o[:, None, :]))
            den = 1.0 - e.sum(axis=1, keepdims=True)
            out[b, a] = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.inf)
    return out


def fp8_tolerance(q_codes, k_codes, v_codes, kind, window=0, scale=None, rows=None,
                  exact_weights=False, bf16_output=True, rounded_denominator=False, fmt="e4m3"):
    """Per-element bound (float64, shaped like the output) on |O_kernel -
    O_exact|: the E4M3 rounding of P (``fp8_error_bound``, left out when
    ``exact_weights``), the fp32 score, exponent and accumulation errors and,
    when ``bf16_output``, the bf16 rounding of the output (derivation in the
    module docstring).  ``rounded_denominator``: the kernel sums the
    denominator from the rounded weights on the matrix cores.  ``fmt``: the
    input format of the codes."""
    q = fp8_decode(q_codes, fmt)
    k = fp8_decode(k_codes, fmt)
    v = fp8_decode(v_codes, fmt)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    c = abs(float(scale)) / np.log(2.0)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    vis = reference.visibility(rows, S, kind, window)
    n_vis = vis.sum(axis=1, keepdims=True).astype(np.float64)
    exact = reference.attention(q, k, v, kind, window, (), scale=scale, rows=rows)
    b = np.zeros_like(exact) if exact_weights else \
        fp8_error_bound(q_codes, k_codes, v_codes, kind, window, scale, rows, rounded_denominator,
                        fmt)
    den_chain = (n_vis / 16 + 48) if rounded_denominator else (n_vis + 8)
    out = np.empty_like(exact)
    for bb in range(B):
        for a in range(Hq):
            h = reference.kv_head(a, Hq, Hkv)
            w = reference.weights(q[bb, a, rows], k[bb, h], rows, kind, window, (), scale)
            mean_abs = w @ np.abs(v[bb, h])               # sum_j p_j |v_j| / L
            if exact_weights:
                ew = np.zeros((rows.size, 1))
            else:
                amag = np.where(vis, np.abs(q[bb, a, rows]) @ np.abs(k[bb, h]).T, 0.0)
                ew = np.log(2.0) * (D + 4) * U_F32 * c * amag.max(axis=1, keepdims=True) \
                    + 2 * U_F32
            f = (2 * ew * (1 + 2 * ew) + (n_vis / 16 + 48) * U_F32) * mean_abs \
                + den_chain * U_F32 * np.abs(exact[bb, a])
            out[bb, a] = b[bb, a] + f
    if bf16_output:
        out = out + U_BF16 * (np.abs(exact) + out)
    return out
