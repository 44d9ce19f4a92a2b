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
arithmetic it does (first order in the fp32 unit u = 2^-24).  The FP8 matrix
instruction does not sum its 64 products exactly: measured on the hardware
(an in-bounds probe of the instruction), it splits them into groups of 8
consecutive reduction indices and truncates each product toward zero to a
multiple of 2^(E - 13), E the exponent of the group's largest product
(floor of log2 of its magnitude); the truncated products are then summed
and added to the fp32 accumulator.  A product of two FP8 values has at most
8 significant bits, so the group's largest product is exact and each of the
other seven loses less than one grid step: a group's error is below
U_MFMA = 7 * 2^-13 times its largest product, and an instruction's error below
U_MFMA times the sum of its groups' largest products.

* Scores and exponent.  A score is a sum of D products in D / 64
  instructions, D / 8 groups; its truncation error is below U_MFMA T_j, T_j
  the sum of the groups' largest |q_d k_jd|, which is at most both A_j =
  sum_d |q_d k_jd| and (D / 8) max_d |q_d| max_d |k_jd| (whatever the
  grouping); the fp32 additions add at most D u A_j.  The exponent argument
  x = s c - m c (c = |scale| log2 e, rounded to fp32) adds at most
  4 u c max(A), so |dx| <= c max_j (U_MFMA min(A_j, (D/8) max|q| max|k_j|)
  + (D + 4) u A_j), and 2^x with v_exp_f32 (about one ulp) gives each weight
  a relative error of at most ew = ln2 |dx| + 2 u.  Relative weight errors of
  at most ew move a weighted mean by at most 2 ew (1 + 2 ew) sum_j p_j |v_j|
  / L.
* Accumulation.  The numerator sum_j p~_j v_j: the instructions' truncation,
  below U_MFMA sum_j p_j |v_j| / L (every group's largest product is one of
  the terms); with all queries zero the weights are exactly 1 and the
  products are the values themselves, so the truncation is bounded per key
  instead: v_j loses nothing when it is a multiple of g* = 2^(E - 13), E the
  binade of the largest visible |v| (no group's grid is coarser), and less
  than min(|v_j|, g*) otherwise.  Then the chain of fp32 additions of
  partial sums, taken as at
  most 16 keys each (n_vis / 16 + 1 steps, plus rescales and the final
  division), error <= (n_vis / 16 + 48) u sum_j p_j |v_j| / L.  The
  denominator summed by the vector ALUs is a chain of at most n_vis fp32
  additions of positive weights, relative error <= (n_vis + 8) u; summed on
  the matrix cores (the rounded weights times ones) it is a chain of the
  numerator's kind plus the truncation, relative error <= (n_vis / 16 + 48) u
  + U_MFMA (no truncation when the weights are exactly 1); either moves O by
  that fraction of |O|.
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
MFMA_GROUP = 8              # products per truncation group of the FP8 instruction
MFMA_GRID_BITS = 13         # the group's grid: 2^-13 of its largest product's binade


def u_mfma():
    """A group's truncation error per unit of its largest product: at most
    7 of its 8 products lose less than one grid step each."""
    return (MFMA_GROUP - 1) * 2.0 ** -MFMA_GRID_BITS


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


def fp8_attention(q_codes, k_codes, v_codes, kind, window=0, scale=None, rows=None, fmt="e4m3",
                  global_idx=()):
    """Exact masked attention (float64) on the decoded FP8 inputs (global_idx:
    the global positions of "local_global")."""
    return reference.attention(fp8_decode(q_codes, fmt), fp8_decode(k_codes, fmt),
                               fp8_decode(v_codes, fmt), kind, window, global_idx, scale=scale,
                               rows=rows)


def fp8_error_bound(q_codes, k_codes, v_codes, kind, window=0, scale=None, rows=None,
                    rounded_denominator=False, fmt="e4m3", global_idx=()):
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
            w = reference.weights(q[b, a, rows], k[b, h], rows, kind, window, global_idx, scale)
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
                  exact_weights=False, bf16_output=True, rounded_denominator=False, fmt="e4m3",
                  global_idx=()):
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
    vis = reference.visibility(rows, S, kind, window, global_idx)
    n_vis = vis.sum(axis=1, keepdims=True).astype(np.float64)
    exact = reference.attention(q, k, v, kind, window, global_idx, scale=scale, rows=rows)
    b = np.zeros_like(exact) if exact_weights else \
        fp8_error_bound(q_codes, k_codes, v_codes, kind, window, scale, rows, rounded_denominator,
                        fmt, global_idx)
    um = u_mfma()
    den_rel = (n_vis + 8) * U_F32
    if rounded_denominator:
        den_rel = (n_vis / 16 + 48) * U_F32 + (0.0 if exact_weights else um)
    out = np.empty_like(exact)
    for bb in range(B):
        for a in range(Hq):
            h = reference.kv_head(a, Hq, Hkv)
            w = reference.weights(q[bb, a, rows], k[bb, h], rows, kind, window, global_idx, scale)
            mean_abs = w @ np.abs(v[bb, h])               # sum_j p_j |v_j| / L
            if exact_weights:
                ew = np.zeros((rows.size, 1))
                vv = np.abs(v[bb, h])
                top = np.where(vis, vv.max(axis=1)[None, :], 0.0).max(axis=1, keepdims=True)
                g = np.exp2(np.floor(np.log2(np.where(top > 0, top, 1.0))) - MFMA_GRID_BITS)
                # per row: sum over visible keys of min(|v|, g*) where v is off the grid
                trunc = np.empty((rows.size, D))
                for r in range(rows.size):
                    vr = vv[vis[r]]
                    off = np.mod(vr, g[r, 0]) != 0
                    trunc[r] = np.where(off, np.minimum(vr, g[r, 0]), 0.0).sum(axis=0)
                trunc = trunc / np.maximum(n_vis, 1.0)
            else:
                amag = np.where(vis, np.abs(q[bb, a, rows]) @ np.abs(k[bb, h]).T, 0.0)
                tops = (D / MFMA_GROUP) * np.outer(np.abs(q[bb, a, rows]).max(axis=1),
                                                   np.abs(k[bb, h]).max(axis=1))
                ds = np.where(vis, um * np.minimum(amag, tops) + (D + 4) * U_F32 * amag, 0.0)
                ew = np.log(2.0) * c * ds.max(axis=1, keepdims=True) + 2 * U_F32
                trunc = um * mean_abs
            f = (2 * ew * (1 + 2 * ew) + (n_vis / 16 + 48) * U_F32) * mean_abs + trunc \
                + den_rel * np.abs(exact[bb, a])
            out[bb, a] = b[bb, a] + f
    if bf16_output:
        out = out + U_BF16 * (np.abs(exact) + out)
    return out
