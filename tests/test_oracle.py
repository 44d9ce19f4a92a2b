"""Pins for the fp64 oracle (CPU only).

Each pin ties the oracle to something other than itself: values printed on the
pages (fixtures under tests/golden/), closed forms, invariants the pages state,
torch's CPU attention routine as an independent library implementation, and a
pure-Python loop on tiny inputs.  ``test_planted_mistakes_are_caught`` plants
plausible mistakes in the oracle (on the CPU) and checks that some pin fails
for each.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as oracle_mod
from tests import golden

RNG = np.random.default_rng(12345)


def randn(*shape, rng=None):
    rng = RNG if rng is None else rng
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# independent helpers (no oracle code)
# ----------------------------------------------------------------------------

def torch_mask(S, kind, window=0, globals_=()):
    """Boolean [S, S] mask built from torch's triangular routines."""
    ones = torch.ones(S, S, dtype=torch.bool)
    if kind == "full":
        return ones
    if kind == "causal":
        return torch.tril(ones)
    if kind == "causal_window":
        # j <= i and j >= i - (window - 1)
        return torch.tril(ones) & torch.triu(ones, diagonal=-(window - 1))
    if kind == "local_global":
        m = torch.triu(ones, diagonal=-window) & torch.tril(ones, diagonal=window)
        for g in set(globals_):
            m[g, :] = True
            m[:, g] = True
        return m
    raise ValueError(kind)


def torch_sdpa(q, k, v, kind, window=0, globals_=(), scale=None):
    """torch's CPU scaled_dot_product_attention in float64 with grouped heads."""
    S, D = q.shape[2], q.shape[3]
    m = torch_mask(S, kind, window, globals_)
    tq, tk, tv = (torch.from_numpy(np.asarray(x, dtype=np.float64)) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, scale=(1.0 / math.sqrt(D) if scale is None else scale),
        enable_gqa=True)
    return out.numpy()


def brute_force(q, k, v, kind, window=0, globals_=(), scale=None):
    """Scalar loops with math.exp / math.fsum on tiny inputs."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    gs = set(globals_)
    out = np.zeros(q.shape)
    for b in range(B):
        for a in range(Hq):
            h = a // group
            for i in range(S):
                vis = []
                for j in range(S):
                    if kind == "full":
                        ok = True
                    elif kind == "causal":
                        ok = j <= i
                    elif kind == "causal_window":
                        ok = i - window < j <= i
                    else:
                        ok = abs(i - j) <= window or i in gs or j in gs
                    if ok:
                        vis.append(j)
                s = [scale * math.fsum(float(q[b, a, i, d]) * float(k[b, h, j, d]) for d in range(D))
                     for j in vis]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = math.fsum(e)
                for d in range(D):
                    out[b, a, i, d] = math.fsum(e[t] * float(v[b, h, j, d])
                                                for t, j in enumerate(vis)) / tot
    return out


def rows_closed_form(S, kind, window=0, globals_=()):
    """Visible keys per query row, from closed forms."""
    i = np.arange(S)
    if kind == "full":
        return np.full(S, S)
    if kind == "causal":
        return i + 1
    if kind == "causal_window":
        return np.minimum(i + 1, window)
    g = sorted(set(globals_))
    band = np.minimum(i, window) + np.minimum(S - 1 - i, window) + 1
    extra = np.array([sum(1 for x in g if abs(x - r) > window) for r in range(S)])
    cnt = band + extra
    cnt[g] = S
    return cnt


# ----------------------------------------------------------------------------
# pins (plain functions so the planted-mistake test can rerun them)
# ----------------------------------------------------------------------------

def pin_page_softmax_example():
    fx = golden.load("softmax_example.txt")
    q = np.array(fx["query"][0], dtype=np.float64)
    keys = np.array(fx["key"], dtype=np.float64)
    assert list((keys @ q).astype(int)) == fx["dots"][0]
    # one head, S = 3 keys; the page's scale is sqrt(d_k) = 1; full visibility.
    w = oracle.weights(np.tile(q, (3, 1)), keys, [0, 1, 2], "full", scale=1.0)[0]
    printed = sorted(fx["printed_weights"][0])
    dec = fx["printed_decimals"][0][0]
    assert np.allclose(sorted(np.round(w, dec)), printed, atol=0.5 * 10 ** -dec + 1e-12)
    assert int(np.argmax(w)) + 1 == fx["top_key"][0][0]
    # the same weights reach the output when V is the identity
    o = oracle.attention(np.tile(q, (1, 1, 3, 1)), keys[None, None], np.eye(3)[None, None],
                         "full", scale=1.0)
    assert np.allclose(o[0, 0, 0], w, atol=1e-15)


def pin_page_ranking_example():
    fx = golden.load("ranking_example.txt")
    q = np.array(fx["query"][0], dtype=np.float64)
    keys = np.array(fx["key"], dtype=np.float64)
    w = oracle.weights(np.tile(q, (3, 1)), keys, [0, 1, 2], "full", scale=1.0)[0]
    order = [int(x) + 1 for x in np.argsort(-w)]
    assert order == fx["ranking"][0]


def pin_page_window_example():
    fx = golden.load("window_example.txt")
    w = fx["window"][0][0]
    i = fx["query"][0][0]
    vis = oracle.visibility([i], 32, "local_global", w, ())[0]
    assert list(np.flatnonzero(vis)) == list(range(fx["visible_first"][0][0],
                                                    fx["visible_last"][0][0] + 1))
    assert vis.sum() == 2 * w + 1


def pin_page_longformer_example():
    fx = golden.load("longformer_example.txt")
    S = fx["S"][0][0]
    w = fx["window"][0][0]
    g = fx["globals"][0]
    i = fx["query"][0][0]
    vis = oracle.visibility([i, fx["global_query"][0][0]], S, "local_global", w, g)
    band = set(range(fx["band_first"][0][0], fx["band_last"][0][0] + 1))
    assert set(np.flatnonzero(vis[0])) == band | set(g)
    assert vis[1].all()


def pin_rows_sum_to_one():
    for kind, w, g in (("full", 0, ()), ("causal", 0, ()), ("causal_window", 3, ()),
                       ("local_global", 2, (0, 9))):
        S, D = 17, 5
        q, k = randn(S, D), randn(S, D)
        p = oracle.weights(q, k, np.arange(S), kind, w, g)
        assert np.all(p >= 0)
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
        assert np.all(p[~oracle.visibility(np.arange(S), S, kind, w, g)] == 0.0)


def pin_visible_counts_closed_form():
    cases = [(1, "causal", 0, ()), (7, "causal", 0, ()), (200, "causal_window", 1, ()),
             (200, "causal_window", 37, ()), (200, "causal_window", 250, ()),
             (200, "local_global", 0, ()), (200, "local_global", 13, (0, 5, 77, 199)),
             (200, "local_global", 300, (4,)), (64, "full", 0, ())]
    for S, kind, w, g in cases:
        vis = oracle.visibility(np.arange(S), S, kind, w, g)
        assert np.array_equal(vis.sum(axis=1), rows_closed_form(S, kind, w, g)), (S, kind, w, g)


def pin_workload_pair_totals():
    # exact visible-pair totals per head for the five workloads (closed forms)
    assert oracle.visible_pair_count(256, "causal") == 256 * 257 // 2 == 32896
    assert oracle.visible_pair_count(2048, "causal") == 2048 * 2049 // 2
    assert oracle.visible_pair_count(8192, "causal") == 8192 * 8193 // 2 == 33558528
    w = 4096
    assert oracle.visible_pair_count(16384, "causal_window", w) == \
        w * (w + 1) // 2 + (16384 - w) * w == 58722304
    cf = int(rows_closed_form(8192, "local_global", 512, (0, 1000, 3000, 6000)).sum())
    assert oracle.visible_pair_count(8192, "local_global", 512, (0, 1000, 3000, 6000)) == cf \
        == 8192492


def count_products_brute_force(S, D, kind, window=0, g=()):
    """Pure-Python forward of one head on tiny inputs that counts the
    floating-point multiplies and adds of its two products: every score is a
    D-term dot product (D multiplies, D adds into a zero accumulator) and every
    visible key adds its weighted value row to the output (D multiplies, D
    adds).  The softmax's exp, max and sum are not counted.  Visibility is
    written out here from the mask definitions, not taken from the oracle."""
    rng = np.random.default_rng(S * 31 + D)
    q = rng.standard_normal((S, D)).tolist()
    k = rng.standard_normal((S, D)).tolist()
    v = rng.standard_normal((S, D)).tolist()
    ops = 0
    for i in range(S):
        vis = []
        for j in range(S):
            if kind == "full":
                ok = True
            elif kind == "causal":
                ok = j <= i
            elif kind == "causal_window":
                ok = i - window < j <= i
            else:
                ok = abs(i - j) <= window or i in g or j in g
            if ok:
                vis.append(j)
        scores = []
        for j in vis:
            acc = 0.0
            for d in range(D):
                acc = acc + q[i][d] * k[j][d]
                ops += 2
            scores.append(acc)
        m = max(scores)
        w = [math.exp(x - m) for x in scores]
        tot = math.fsum(w)
        out = [0.0] * D
        for wj, j in zip(w, vis):
            for d in range(D):
                out[d] = out[d] + (wj / tot) * v[j][d]
                ops += 2
    return ops


def pin_effective_flops():
    # "Transformer 演进与变体", section 前馈网络效率: the score product and the
    # output product of full attention are n^2 d multiply-adds each; two FLOPs
    # per multiply-add, per query head and batch entry
    for n, d in ((64, 16), (300, 128)):
        assert oracle.effective_flops(1, 1, n, d, "full") == 2 * (n * n * d + n * n * d)
        assert oracle.effective_flops(3, 5, n, d, "full") == 15 * 2 * (2 * n * n * d)
    # operation counts of a pure-Python forward on tiny shapes, every mask kind
    for kind, w, g in (("full", 0, ()), ("causal", 0, ()), ("causal_window", 3, ()),
                       ("local_global", 2, (0, 9))):
        S, D = 13, 5
        assert oracle.effective_flops(1, 1, S, D, kind, w, g) == \
            count_products_brute_force(S, D, kind, w, g), kind
        assert oracle.effective_flops(2, 3, S, D, kind, w, g) == \
            6 * count_products_brute_force(S, D, kind, w, g), kind
    # the five workloads' totals (independently tabulated: 3.369e7, 1.375e11,
    # 549,822,922,752, 9.621e11, 2.517e10)
    assert oracle.effective_flops(1, 4, 256, 64, "causal") == 33685504
    assert oracle.effective_flops(4, 32, 2048, 128, "causal") == 137506062336
    assert oracle.effective_flops(1, 32, 8192, 128, "causal") == 549822922752
    assert oracle.effective_flops(1, 32, 16384, 128, "causal_window", 4096) == 962106228736
    assert oracle.effective_flops(1, 12, 8192, 64, "local_global", 512,
                                  (0, 1000, 3000, 6000)) == 25167335424


def pin_only_global_rows_see_everything():
    S, w, g = 8192, 512, (0, 1000, 3000, 6000)
    cnt = rows_closed_form(S, "local_global", w, g)
    vis_rows = np.arange(0, S, 97).tolist() + list(g)
    vis = oracle.visibility(vis_rows, S, "local_global", w, g)
    for r, row in zip(vis_rows, vis):
        assert (row.sum() == S) == (r in g)
        assert row.sum() == cnt[r]
    assert cnt[[r for r in range(S) if r not in g]].max() <= 2 * w + 1 + len(g)


def pin_window_ge_S_equals_causal():
    S, D = 23, 6
    q, k, v = randn(1, 2, S, D), randn(1, 2, S, D), randn(1, 2, S, D)
    a = oracle.attention(q, k, v, "causal")
    for w in (S, S + 5, 10 * S):
        assert np.array_equal(oracle.attention(q, k, v, "causal_window", w), a)


def pin_identical_keys_give_mean_of_visible_values():
    S, D = 19, 4
    q, v = randn(1, 1, S, D), randn(1, 1, S, D)
    k = np.broadcast_to(randn(D), (1, 1, S, D)).copy()
    for kind, w, g in (("causal", 0, ()), ("causal_window", 4, ()), ("local_global", 3, (7,)),
                       ("full", 0, ())):
        o = oracle.attention(q, k, v, kind, w, g)
        vis = oracle.visibility(np.arange(S), S, kind, w, g)
        for i in range(S):
            assert np.allclose(o[0, 0, i], v[0, 0, vis[i]].mean(axis=0), atol=1e-12)


def pin_closed_form_rows():
    S, D = 16, 8
    q, k, v = randn(2, 3, S, D), randn(2, 3, S, D), randn(2, 3, S, D)
    # causal row 0 sees only key 0
    assert np.allclose(oracle.attention(q, k, v, "causal")[:, :, 0], v[:, :, 0], atol=1e-14)
    # window of one key sees only itself
    assert np.allclose(oracle.attention(q, k, v, "causal_window", 1), v, atol=1e-14)
    # band of radius zero, no globals
    assert np.allclose(oracle.attention(q, k, v, "local_global", 0), v, atol=1e-14)
    # zero scale gives uniform weights: running mean of V under the causal mask
    cm = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    assert np.allclose(oracle.attention(q, k, v, "causal", scale=0.0), cm, atol=1e-12)
    # a single dominant key: with a huge score the output is that key's value row
    k2 = k.copy()
    k2[:, :, 5] = 1e3 * q[:, :, 9]
    o = oracle.attention(q, k2, v, "full")
    assert np.allclose(o[:, :, 9], v[:, :, 5], atol=1e-9)


def pin_grouped_heads():
    S, D = 12, 4
    B, Hq = 2, 4
    q = randn(B, Hq, S, D)
    for Hkv in (1, 2, 4):
        k, v = randn(B, Hkv, S, D), randn(B, Hkv, S, D)
        G = Hq // Hkv
        # repeating each KV head G times (consecutive query heads) gives plain multi-head
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        for kind, w, g in (("causal", 0, ()), ("local_global", 2, (3,))):
            a = oracle.attention(q, k, v, kind, w, g)
            assert np.array_equal(a, oracle.attention(q, kr, vr, kind, w, g))
            assert np.allclose(a, torch_sdpa(q, k, v, kind, w, g), atol=1e-12)


def pin_permutation_equivariance():
    S, D = 15, 6
    q, k, v = randn(1, 1, S, D), randn(1, 1, S, D), randn(1, 1, S, D)
    perm = RNG.permutation(S)
    a = oracle.attention(q, k, v, "full")
    b = oracle.attention(q[:, :, perm], k[:, :, perm], v[:, :, perm], "full")
    assert np.allclose(a[:, :, perm], b, atol=1e-12)


def pin_causality_perturbation():
    S, D, i0 = 30, 5, 11
    q, k, v = randn(1, 2, S, D), randn(1, 2, S, D), randn(1, 2, S, D)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i0 + 1:] = randn(1, 2, S - i0 - 1, D)
    v2[:, :, i0 + 1:] = randn(1, 2, S - i0 - 1, D)
    for kind, w in (("causal", 0), ("causal_window", 6)):
        a = oracle.attention(q, k, v, kind, w)
        b = oracle.attention(q, k2, v2, kind, w)
        assert np.array_equal(a[:, :, :i0 + 1], b[:, :, :i0 + 1])
        assert not np.allclose(a[:, :, i0 + 1:], b[:, :, i0 + 1:])


def pin_torch_sdpa_crosscheck():
    for (Hq, Hkv), (kind, w, g), S in zip(
            [(1, 1), (4, 1), (4, 2), (4, 4), (6, 3), (8, 2)],
            [("full", 0, ()), ("causal", 0, ()), ("causal_window", 5, ()),
             ("local_global", 4, (0, 17, 40)), ("local_global", 0, (63,)),
             ("causal_window", 64, ())],
            [33, 64, 65, 41, 64, 100]):
        D = 8
        q, k, v = randn(2, Hq, S, D), randn(2, Hkv, S, D), randn(2, Hkv, S, D)
        for scale in (None, 0.3):
            a = oracle.attention(q, k, v, kind, w, g, scale=scale, block_rows=16)
            b = torch_sdpa(q, k, v, kind, w, g, scale=scale)
            assert np.allclose(a, b, atol=1e-12), (Hq, Hkv, kind)


def pin_brute_force_tiny():
    for (Hq, Hkv) in [(1, 1), (4, 1), (4, 2), (4, 4)]:
        for kind, w, g in (("full", 0, ()), ("causal", 0, ()), ("causal_window", 3, ()),
                           ("local_global", 1, (2, 5))):
            for S, D in ((1, 3), (6, 3), (9, 8)):
                if any(x >= S for x in g):
                    g = tuple(x for x in g if x < S)
                q, k, v = randn(1, Hq, S, D), randn(1, Hkv, S, D), randn(1, Hkv, S, D)
                a = oracle.attention(q, k, v, kind, w, g)
                b = brute_force(q, k, v, kind, w, g)
                assert np.allclose(a, b, atol=1e-13, rtol=0), (Hq, Hkv, kind, S, D)


def pin_sampled_rows_match_full():
    S, D = 50, 4
    q, k, v = randn(1, 2, S, D), randn(1, 1, S, D), randn(1, 1, S, D)
    full = oracle.attention(q, k, v, "causal_window", 7)
    rows = [49, 0, 13, 13, 31]
    part = oracle.attention(q, k, v, "causal_window", 7, rows=rows)
    assert np.array_equal(part, full[:, :, rows])


def online_softmax_attention(q, k, v, mask, scale, block, lazy):
    """Blockwise online softmax in float64 ("Transformer 演进与变体", section
    Flash Attention: per key block update the running maximum m, rescale the
    running denominator l and the accumulator by exp(m_old - m_new), add the
    block's exp(s - m_new)).  With lazy > 0 the reference maximum moves only
    when the block maximum exceeds it by more than lazy (natural-log units),
    the variant the GPU kernels use; the result must not change."""
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        for a in range(Hq):
            qa, ka, va = q[b, a], k[b, a // G], v[b, a // G]
            m = np.full(S, -np.inf)
            l = np.zeros(S)
            acc = np.zeros((S, D))
            for j0 in range(0, S, block):
                s = scale * (qa @ ka[j0:j0 + block].T)
                s[~mask[:, j0:j0 + block]] = -np.inf
                bmax = s.max(axis=1)
                move = bmax > m + lazy
                m_new = np.where(move, bmax, m)
                with np.errstate(invalid="ignore"):  # -inf - -inf, discarded by the where
                    alpha = np.where(np.isneginf(m_new), 1.0, np.exp(m - m_new))
                    p = np.where(np.isneginf(s), 0.0, np.exp(s - m_new[:, None]))
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ va[j0:j0 + block]
                m = m_new
            out[b, a] = acc / l[:, None]
    return out


def pin_online_softmax_recurrence():
    for kind, w, g in (("full", 0, ()), ("causal", 0, ()), ("causal_window", 5, ()),
                       ("local_global", 3, (0, 17, 30))):
        S, D = 37, 8
        q, k, v = randn(2, 4, S, D), randn(2, 2, S, D), randn(2, 2, S, D)
        q[0, 1, 5] *= 40.0  # a row whose block maxima jump far above the first block's
        mask = torch_mask(S, kind, w, g).numpy()
        ref = oracle.attention(q, k, v, kind, w, g, scale=0.35)
        for block in (1, 7, 16, 64):
            for lazy in (0.0, 8.0 * math.log(2.0)):
                got = online_softmax_attention(q, k, v, mask, 0.35, block, lazy)
                assert np.allclose(got, ref, atol=1e-12, rtol=0), (kind, block, lazy)


PINS = [
    pin_page_softmax_example,
    pin_page_ranking_example,
    pin_page_window_example,
    pin_page_longformer_example,
    pin_rows_sum_to_one,
    pin_visible_counts_closed_form,
    pin_workload_pair_totals,
    pin_effective_flops,
    pin_only_global_rows_see_everything,
    pin_window_ge_S_equals_causal,
    pin_identical_keys_give_mean_of_visible_values,
    pin_closed_form_rows,
    pin_grouped_heads,
    pin_permutation_equivariance,
    pin_causality_perturbation,
    pin_torch_sdpa_crosscheck,
    pin_brute_force_tiny,
    pin_sampled_rows_match_full,
    pin_online_softmax_recurrence,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# the oracle's own argument checks
# ----------------------------------------------------------------------------

def test_rejects_bad_arguments():
    q = randn(1, 2, 4, 3)
    k = randn(1, 2, 4, 3)
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, "local_global", 1, (4,))  # global out of range
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, "causal_window", 0)
    with pytest.raises(ValueError):
        oracle.attention(q, randn(1, 3, 4, 3), randn(1, 3, 4, 3), "full")  # 2 % 3
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, "nope")


def test_global_set_semantics():
    S = 40
    a = oracle.visibility(np.arange(S), S, "local_global", 2, (5, 30, 5, 0))
    b = oracle.visibility(np.arange(S), S, "local_global", 2, (0, 5, 30))
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

def _orig(name):
    return getattr(oracle_mod, name)


def _mut_causal_strict(rows, S, kind, window=0, global_idx=()):
    vis = _ORIG_VIS(rows, S, kind, window, global_idx)
    if kind == "causal":
        i = np.asarray(rows)[:, None]
        j = np.arange(S)[None, :]
        vis = vis & (j != i) | ((i == 0) & (j == 0))  # drops the diagonal except row 0
    return vis


def _mut_window_off_by_one(rows, S, kind, window=0, global_idx=()):
    if kind == "causal_window":
        i = np.asarray(rows)[:, None]
        j = np.arange(S)[None, :]
        return (j <= i) & (j >= i - window)
    return _ORIG_VIS(rows, S, kind, window, global_idx)


def _mut_band_one_sided(rows, S, kind, window=0, global_idx=()):
    if kind == "local_global":
        i = np.asarray(rows)[:, None]
        j = np.arange(S)[None, :]
        g = oracle_mod.global_set(global_idx, S)
        return ((j - i <= window) & (j <= i)) | np.isin(i, g) | np.isin(j, g)
    return _ORIG_VIS(rows, S, kind, window, global_idx)


def _mut_globals_columns_only(rows, S, kind, window=0, global_idx=()):
    if kind == "local_global":
        i = np.asarray(rows)[:, None]
        j = np.arange(S)[None, :]
        g = oracle_mod.global_set(global_idx, S)
        return (np.abs(i - j) <= window) | np.isin(j, g)
    return _ORIG_VIS(rows, S, kind, window, global_idx)


def _mut_head_map_modulo(a, Hq, Hkv):
    return a % Hkv


def _mut_softmax_no_normalise(scores):
    m = scores.max(axis=1, keepdims=True)
    return np.exp(scores - m)


def _mut_softmax_wrong_sign(scores):
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(m - scores)
    e[~np.isfinite(scores)] = 0.0
    return e / e.sum(axis=1, keepdims=True)


_ORIG_VIS = oracle_mod.visibility
_ORIG_WEIGHTS = oracle_mod.weights


def _mut_scale_ignored(q_rows, k, rows, kind, window=0, global_idx=(), scale=None):
    return _ORIG_WEIGHTS(q_rows, k, rows, kind, window, global_idx, scale=1.0)


def _mut_transposed_scores(q_rows, k, rows, kind, window=0, global_idx=(), scale=None):
    # scores taken as K Q^T restricted to the same rows (an operand-order mistake)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S, D = k.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    s = scale * (k[np.asarray(rows)] @ q_rows.T) if len(rows) == S else scale * (q_rows @ k.T)
    vis = _ORIG_VIS(rows, S, kind, window, global_idx)
    return oracle_mod.softmax_rows(np.where(vis, s, -np.inf))


def _mut_flops_two_d(B, Hq, S, D, kind, window=0, global_idx=()):
    # one product counted, or multiply-adds counted as one FLOP
    return 2 * D * oracle_mod.visible_pair_count(S, kind, window, global_idx) * B * Hq


MUTATIONS = {
    "causal_drops_diagonal": ("visibility", _mut_causal_strict),
    "window_off_by_one": ("visibility", _mut_window_off_by_one),
    "band_one_sided": ("visibility", _mut_band_one_sided),
    "global_rows_not_dense": ("visibility", _mut_globals_columns_only),
    "head_map_modulo": ("kv_head", _mut_head_map_modulo),
    "softmax_not_normalised": ("softmax_rows", _mut_softmax_no_normalise),
    "softmax_wrong_sign": ("softmax_rows", _mut_softmax_wrong_sign),
    "scale_ignored": ("weights", _mut_scale_ignored),
    "scores_transposed": ("weights", _mut_transposed_scores),
    "flops_two_d": ("effective_flops", _mut_flops_two_d),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(oracle_mod, attr, fn)
    # the package re-exports; patch those names too so pins see the mutation
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {mutation}"
