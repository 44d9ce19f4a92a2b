"""fp64 CPU oracle for block-sparse attention patterns.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP path (whose layouts come from its own C builders; the
tests compare the two bit for bit) and none with the other oracle modules.

What it computes -- "第 8 章 AI 算法Transformer大模型", section 8.3 (sparse and
linear attention):

* Strided pattern (section 8.3.1, Sparse Transformer): a query looks at the
  positions just before it (a local window of k) and at the positions l, 2l,
  3l, ... before it.
* Fixed pattern (section 8.3.1): the sequence is cut into blocks; a query
  looks at every position of its own block and, in the earlier blocks, at the
  positions in the same column as itself.
* Big Bird (section 8.3.3): each query looks at w neighbours, at r randomly
  chosen positions and at g global positions; the global positions look at
  every position.
* Section 8.3.4 notes that these patterns run as block-sparse matrix products
  in practice (Big Bird's kernel).

Readings taken where the pages leave it open:

* Every pattern is applied to BLOCKS of `block` positions (the block-sparse
  form the page names): the layout is a boolean [nb][nb] matrix over query
  blocks I and key blocks J, nb = ceil(S / block), and position j is visible
  from query i when layout[i // block][j // block] holds (and, for a causal
  call, j <= i; and j < S).  A query's own block is always in the layout, so
  a query sees itself.
* Strided (local k_b, stride l_b, both in blocks): J <= I with I - J <= k_b,
  or I - J a positive multiple of l_b.
* Fixed (chunk c, in blocks: the page's "block" is a chunk of c layout
  blocks, its "column" the position of a block inside its chunk): J <= I in
  the same chunk (J // c == I // c), or J < I in the same column
  (J % c == I % c).
* Big Bird (radius w_b, g global blocks, random blocks as an INPUT array
  rand[I][0..r-1] since the pages fix no generator): |I - J| <= w_b, or J in
  rand[I], or J < g, or I < g.
* A query row that sees no key has output zero.

Layout: q [B][Hq][S][D], k and v [B][Hkv][S][D], query head a reads key/value
head a // (Hq / Hkv).  float64 on the exact inputs.

Pinned by tests/test_oracle_sparse.py.
"""
from __future__ import annotations

import numpy as np


def n_blocks(S, block):
    return -(-S // block)


def strided_layout(nb, local, stride):
    """Sparse Transformer strided pattern over nb blocks (causal)."""
    if local < 0 or stride < 1:
        raise ValueError("local >= 0 and stride >= 1")
    lay = np.zeros((nb, nb), dtype=bool)
    for I in range(nb):
        for J in range(I + 1):
            d = I - J
            lay[I, J] = d <= local or d % stride == 0
    return lay


def fixed_layout(nb, chunk):
    """Sparse Transformer fixed pattern over nb blocks (causal)."""
    if chunk < 1:
        raise ValueError("chunk >= 1")
    lay = np.zeros((nb, nb), dtype=bool)
    for I in range(nb):
        for J in range(I + 1):
            lay[I, J] = J // chunk == I // chunk or J % chunk == I % chunk
    return lay


def bigbird_layout(nb, radius, n_global, rand_blocks):
    """Big Bird pattern over nb blocks: window, random blocks (input), global."""
    rand_blocks = np.asarray(rand_blocks, dtype=np.int64).reshape(nb, -1)
    lay = np.zeros((nb, nb), dtype=bool)
    for I in range(nb):
        for J in range(nb):
            lay[I, J] = abs(I - J) <= radius or J < n_global or I < n_global
        for J in rand_blocks[I]:
            if not 0 <= J < nb:
                raise ValueError("random block out of range")
            lay[I, J] = True
    return lay


def block_visible(layout, block, causal, S, i):
    """Visible keys of query i as a boolean vector of length S."""
    j = np.arange(S)
    vis = np.asarray(layout, dtype=bool)[i // block][j // block]
    if causal:
        vis = vis & (j <= i)
    return vis


def block_sparse_attention(q, k, v, layout, block, causal, scale=None, rows=None):
    """Attention output, float64, shape [B, Hq, S, D] (or the selected rows)."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    nb = n_blocks(S, block)
    if np.asarray(layout).shape != (nb, nb):
        raise ValueError("layout must be [nb][nb]")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = list(range(S)) if rows is None else [int(i) for i in rows]
    out = np.zeros((B, Hq, len(rows), D), dtype=np.float64)
    for r, i in enumerate(rows):
        vis = block_visible(layout, block, causal, S, i)
        if not vis.any():
            continue
        for b in range(B):
            for a in range(Hq):
                h = a // G
                s = float(scale) * (k[b, h].astype(np.float64) @ q[b, a, i].astype(np.float64))
                s = np.where(vis, s, -np.inf)
                e = np.exp(s - s.max())
                out[b, a, r] = (e / e.sum()) @ v[b, h].astype(np.float64)
    return out


def block_sparse_pairs(S, layout, block, causal):
    """Visible (query, key) pairs of one head."""
    return int(sum(block_visible(layout, block, causal, S, i).sum() for i in range(S)))
