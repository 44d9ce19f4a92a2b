"""fp64 CPU oracle for attention with different query and key counts.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests do.  It shares no code with the HIP path, and none
with the other oracle modules (the tests compare them).

What it computes (plain definition, one query row at a time): q holds Sq query
rows and k, v hold Skv key/value rows of each (batch, head).

* Cross attention -- "Trasformer 浅析", section 交叉注意力: the queries come
  from one sequence and the keys and values from another, so their lengths
  differ; every key is visible ("full").
* A query chunk against a longer prefix -- "Transformer 架构及其变体", section
  预填充创建缓存，解码复用缓存 (a long prompt may be prefilled in chunks; each
  chunk's queries attend to the cached prefix and to themselves causally).

Reading taken where the pages leave it open: the queries are the LAST Sq
positions of the key sequence (aligned at the bottom right), so query i sits
at key position p_i = i + Skv - Sq.  Visibility:

    full           every key j < Skv
    causal         j <= p_i
    causal_window  p_i - w < j <= p_i

A query that sees no key (p_i < 0, which needs Skv < Sq) has output zero.
With Sq == Skv this is the square attention of reference.py.

Layout: q [B][Hq][Sq][D], k and v [B][Hkv][Skv][D] (logical layout; strided
device layouts are a matter of the tests).  float64 on the exact inputs.

Pinned by tests/test_oracle_cross.py.
"""
from __future__ import annotations

import numpy as np

FULL = "full"
CAUSAL = "causal"
CAUSAL_WINDOW = "causal_window"
CROSS_MASK_KINDS = (FULL, CAUSAL, CAUSAL_WINDOW)


def cross_visible_range(Sq, Skv, i, kind, window=0):
    """Visible keys of query i as a half-open range [lo, hi) of key positions."""
    p = i + Skv - Sq
    if kind == FULL:
        return 0, Skv
    if kind == CAUSAL:
        return 0, max(0, min(Skv, p + 1))
    if kind == CAUSAL_WINDOW:
        if window < 1:
            raise ValueError("causal_window needs window >= 1")
        return max(0, p - window + 1), max(0, min(Skv, p + 1))
    raise ValueError(f"unknown mask kind {kind!r}")


def cross_attention(q, k, v, kind, window=0, scale=None, rows=None):
    """Attention output, float64, shape [B, Hq, Sq, D]; with `rows` (query row
    indices) only those rows, shape [B, Hq, len(rows), D]."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Skv, D) or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = list(range(Sq)) if rows is None else [int(i) for i in rows]
    out = np.zeros((B, Hq, len(rows), D), dtype=np.float64)
    for b in range(B):
        for a in range(Hq):
            h = a // G
            for r, i in enumerate(rows):
                lo, hi = cross_visible_range(Sq, Skv, i, kind, window)
                if hi <= lo:
                    continue
                kk = k[b, h, lo:hi].astype(np.float64)
                vv = v[b, h, lo:hi].astype(np.float64)
                s = float(scale) * (kk @ q[b, a, i].astype(np.float64))
                e = np.exp(s - s.max())
                out[b, a, r] = (e / e.sum()) @ vv
    return out


def cross_visible_pairs(Sq, Skv, kind, window=0):
    """Visible (query, key) pairs of one head."""
    tot = 0
    for i in range(Sq):
        lo, hi = cross_visible_range(Sq, Skv, i, kind, window)
        tot += max(0, hi - lo)
    return tot
