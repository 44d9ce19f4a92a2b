"""Pins for the fp64 block-sparse oracle (CPU only).

oracle/sparse.py is tied to: hand-worked layouts of each pattern on eight
blocks (derived from the definitions in its header, written out here as
sets), the square oracle (reference.py) for dense layouts and for the
block-diagonal layout (each block on its own), limits in which a pattern
becomes dense, and a pure-Python loop.  ``test_planted_sparse_mistakes_are_
caught`` plants plausible mistakes and checks that a pin fails for each.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import sparse as sp


def randn(rng, *shape):
    return rng.standard_normal(shape)


def rows_of(lay):
    return [set(int(j) for j in np.nonzero(row)[0]) for row in lay]


def pin_strided_by_hand():
    # local 1, stride 3: own block, the one before, and 3, 6 blocks back
    want = [{0}, {0, 1}, {1, 2}, {0, 2, 3}, {1, 3, 4}, {2, 4, 5}, {0, 3, 5, 6}, {1, 4, 6, 7}]
    assert rows_of(sp.strided_layout(8, 1, 3)) == want
    # local 0, stride 2: own block and every second block back
    want = [{0}, {1}, {0, 2}, {1, 3}, {0, 2, 4}, {1, 3, 5}, {0, 2, 4, 6}, {1, 3, 5, 7}]
    assert rows_of(sp.strided_layout(8, 0, 2)) == want


def pin_fixed_by_hand():
    # chunks of 3 blocks: {0,1,2} {3,4,5} {6,7}; columns = block % 3
    want = [{0}, {0, 1}, {0, 1, 2}, {0, 3}, {1, 3, 4}, {2, 3, 4, 5}, {0, 3, 6}, {1, 4, 6, 7}]
    assert rows_of(sp.fixed_layout(8, 3)) == want


def pin_bigbird_by_hand():
    rand = [[5], [7], [0], [6], [1], [2], [4], [3]]
    lay = sp.bigbird_layout(8, 1, 1, rand)
    want = [set(range(8)),                       # the global block sees everything
            {0, 1, 2, 7}, {0, 1, 2, 3}, {0, 2, 3, 4, 6}, {0, 1, 3, 4, 5},
            {0, 2, 4, 5, 6}, {0, 4, 5, 6, 7}, {0, 3, 6, 7}]
    assert rows_of(lay) == want


def pin_dense_layouts_are_plain_attention():
    rng = np.random.default_rng(30)
    B, Hq, Hkv, S, D, blk = 2, 4, 2, 37, 8, 8
    q, k, v = randn(rng, B, Hq, S, D), randn(rng, B, Hkv, S, D), randn(rng, B, Hkv, S, D)
    nb = sp.n_blocks(S, blk)
    ones = np.ones((nb, nb), dtype=bool)
    for causal, kind in ((True, "causal"), (False, "full")):
        got = sp.block_sparse_attention(q, k, v, ones, blk, causal, scale=0.3)
        ref = oracle.attention(q, k, v, kind, scale=0.3)
        assert np.max(np.abs(got - ref)) < 1e-12, kind
    # patterns that cover every earlier block are causal attention
    for lay in (sp.strided_layout(nb, nb, 1), sp.strided_layout(nb, 0, 1), sp.fixed_layout(nb, nb)):
        got = sp.block_sparse_attention(q, k, v, lay, blk, True)
        assert np.max(np.abs(got - oracle.attention(q, k, v, "causal"))) < 1e-12
    # a window radius of nb blocks is full attention
    lay = sp.bigbird_layout(nb, nb, 0, np.zeros((nb, 1), dtype=int))
    got = sp.block_sparse_attention(q, k, v, lay, blk, False)
    assert np.max(np.abs(got - oracle.attention(q, k, v, "full"))) < 1e-12


def pin_block_diagonal_is_blockwise_attention():
    """Only the own block: each block of positions is an independent sequence
    (causal or full inside), checked with the square oracle per block; the
    ragged last block included."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, S, D, blk = 1, 2, 1, 29, 4, 8
    q, k, v = randn(rng, B, Hq, S, D), randn(rng, B, Hkv, S, D), randn(rng, B, Hkv, S, D)
    nb = sp.n_blocks(S, blk)
    eye = np.eye(nb, dtype=bool)
    for causal, kind in ((True, "causal"), (False, "full")):
        got = sp.block_sparse_attention(q, k, v, eye, blk, causal)
        for I in range(nb):
            a, b = I * blk, min(S, (I + 1) * blk)
            ref = oracle.attention(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], kind,
                                   scale=1.0 / math.sqrt(D))
            assert np.max(np.abs(got[:, :, a:b] - ref)) < 1e-12, (kind, I)


def pin_brute_force_loop():
    """Pure-Python loops on a tiny strided case with a ragged last block."""
    rng = np.random.default_rng(32)
    S, D, blk, scale = 11, 3, 3, 0.8
    q, k, v = randn(rng, 1, 1, S, D), randn(rng, 1, 1, S, D), randn(rng, 1, 1, S, D)
    lay = sp.strided_layout(sp.n_blocks(S, blk), 0, 2)
    got = sp.block_sparse_attention(q, k, v, lay, blk, True, scale=scale)
    for i in range(S):
        js = [j for j in range(i + 1) if (i // blk - j // blk) % 2 == 0]
        s = [scale * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) for j in js]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        for d in range(D):
            want = math.fsum(e[n] * v[0, 0, js[n], d] for n in range(len(js))) / math.fsum(e)
            assert abs(got[0, 0, i, d] - want) < 1e-13


def pin_pair_counts():
    # block diagonal, causal: blk*(blk+1)/2 per full block plus the ragged tail
    eye = np.eye(4, dtype=bool)
    assert sp.block_sparse_pairs(30, eye, 8, True) == 3 * 36 + 6 * 7 // 2
    assert sp.block_sparse_pairs(30, eye, 8, False) == 3 * 64 + 36
    assert sp.block_sparse_pairs(30, np.ones((4, 4), dtype=bool), 8, True) == 30 * 31 // 2


PINS = [pin_strided_by_hand, pin_fixed_by_hand, pin_bigbird_by_hand,
        pin_dense_layouts_are_plain_attention, pin_block_diagonal_is_blockwise_attention,
        pin_brute_force_loop, pin_pair_counts]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_sparse_pin(pin):
    pin()


_STRIDED, _FIXED, _BIGBIRD, _VIS = (sp.strided_layout, sp.fixed_layout, sp.bigbird_layout,
                                    sp.block_visible)


def _strided_no_own_block(nb, local, stride):
    lay = _STRIDED(nb, local, stride)
    np.fill_diagonal(lay, False)
    return lay


def _strided_off_by_one(nb, local, stride):
    lay = np.zeros((nb, nb), dtype=bool)
    for I in range(nb):
        for J in range(I + 1):
            d = I - J
            lay[I, J] = d <= local or (d - 1) % stride == 0
    return lay


def _fixed_column_from_chunk(nb, chunk):
    lay = np.zeros((nb, nb), dtype=bool)
    for I in range(nb):
        for J in range(I + 1):
            lay[I, J] = J // chunk == I // chunk or J // chunk == I % chunk
    return lay


def _bigbird_global_rows_local(nb, radius, n_global, rand):
    lay = _BIGBIRD(nb, radius, n_global, rand)
    for I in range(n_global):
        lay[I] = [abs(I - J) <= radius or J < n_global for J in range(nb)]
    return lay


def _bigbird_no_random(nb, radius, n_global, rand):
    return _BIGBIRD(nb, radius, n_global, np.zeros((nb, 1), dtype=int))


def _vis_no_causal(layout, block, causal, S, i):
    return _VIS(layout, block, False, S, i)


def _vis_block_index_by_query(layout, block, causal, S, i):
    # key blocks looked up with the key's offset from the query
    j = np.arange(S)
    vis = np.asarray(layout, dtype=bool)[i // block][np.abs(i - j) // block]
    return vis & (j <= i) if causal else vis


MUTATIONS = {
    "strided_without_own_block": ("strided_layout", _strided_no_own_block),
    "strided_stride_off_by_one": ("strided_layout", _strided_off_by_one),
    "fixed_column_is_chunk": ("fixed_layout", _fixed_column_from_chunk),
    "bigbird_global_rows_not_global": ("bigbird_layout", _bigbird_global_rows_local),
    "bigbird_random_ignored": ("bigbird_layout", _bigbird_no_random),
    "causal_not_applied_in_block": ("block_visible", _vis_no_causal),
    "block_of_distance": ("block_visible", _vis_block_index_by_query),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_sparse_mistakes_are_caught(monkeypatch, mutation):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(sp, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {mutation}"
