"""fp64 CPU oracle for masked, grouped-query scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path.

What it computes (plain definition, no tiling, no online softmax):

* Scores and weights -- "Trasformer 浅析", section 缩放点积注意力: the score
  of query i against key j is their dot product times a scale (1/sqrt(d_k) by
  default, justified in the section 缩放因子的必要性); each row of scores goes
  through a softmax exp(z_j) / sum_j' exp(z_j') and the output row is the
  weight-averaged value rows.
* Masks -- "Trasformer 浅析", section 掩码与三种架构范式 (causal-mask
  equation): a masked pair gets -inf added to its score, so its weight is
  exactly zero.  Here a masked pair is simply excluded from the row.
  Visibility rules:
    full           every key
    causal         j <= i
    causal_window  i - w < j <= i  (w keys including the query itself; the
                   reading taken for the sliding-window workload)
    local_global   |i - j| <= w, or i is a global token, or j is a global token
                   ("Transformer 演进与变体", section 稀疏注意力: a window of
                   radius w, width 2w+1, plus global tokens that see and are
                   seen by every position)
* Heads -- "Transformer 架构及其变体", section 带显式形状的因果自注意力:
  query head a reads key/value head g(a); with Hq query heads over Hkv
  key/value heads, consecutive groups of Hq/Hkv query heads share one
  key/value head, g(a) = floor(a / (Hq/Hkv)).  Hkv == Hq is multi-head
  attention, Hkv == 1 is multi-query attention ("Transformer 演进与变体",
  section GQA：分组查询注意力).

Layout: q is [B][Hq][S][D], k and v are [B][Hkv][S][D].  All arithmetic is in
float64 on the exact input values.  The only deviation from writing the whole
S x S score matrix at once is that query rows are processed in blocks (each
block still spans all S key columns), which keeps memory bounded at S=16384;
it does not change any value.

Pinned by tests/test_oracle.py (worked examples from the pages, closed forms,
invariants, a brute-force loop, and torch's CPU attention as an independent
library routine).
"""
from __future__ import annotations

import numpy as np

FULL = "full"
CAUSAL = "causal"
CAUSAL_WINDOW = "causal_window"
LOCAL_GLOBAL = "local_global"
MASK_KINDS = (FULL, CAUSAL, CAUSAL_WINDOW, LOCAL_GLOBAL)

DEFAULT_BLOCK_ROWS = 1024


def global_set(global_idx, S):
    """The global tokens as a sorted array of distinct positions (a set: order
    and duplicates do not matter).  Positions outside [0, S) are an error."""
    g = np.unique(np.asarray(list(global_idx), dtype=np.int64))
    if g.size and (g[0] < 0 or g[-1] >= S):
        raise ValueError("global token position outside [0, S)")
    return g


def visibility(rows, S, kind, window=0, global_idx=()):
    """Boolean matrix [len(rows), S]: True where query row i may attend to key j."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    if kind == FULL:
        return np.ones((i.shape[0], S), dtype=bool)
    if kind == CAUSAL:
        return j <= i
    if kind == CAUSAL_WINDOW:
        if window < 1:
            raise ValueError("causal_window needs window >= 1")
        return (j <= i) & (j > i - window)
    if kind == LOCAL_GLOBAL:
        if window < 0:
            raise ValueError("local_global needs window >= 0")
        g = global_set(global_idx, S)
        band = np.abs(i - j) <= window
        row_is_global = np.isin(i, g)
        col_is_global = np.isin(j, g)
        return band | row_is_global | col_is_global
    raise ValueError(f"unknown mask kind {kind!r}")


def kv_head(a, Hq, Hkv):
    """Key/value head read by query head a."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return a // (Hq // Hkv)


def softmax_rows(scores):
    """Row softmax of a score block whose excluded entries are -inf.

    Subtracting the row maximum does not change the result (numerator and
    denominator share the factor); it keeps exp() in range.  Every row must
    have at least one finite entry.
    """
    m = scores.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    e = np.exp(scores - m)
    return e / e.sum(axis=1, keepdims=True)


def weights(q_rows, k, rows, kind, window=0, global_idx=(), scale=None):
    """Attention weights of one head: q_rows [R, D] (query rows `rows`), k [S, D]."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S, D = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    scores = float(scale) * (q_rows @ k.T)
    vis = visibility(rows, S, kind, window, global_idx)
    scores = np.where(vis, scores, -np.inf)
    return softmax_rows(scores)


def attention(q, k, v, kind, window=0, global_idx=(), scale=None, rows=None,
              block_rows=DEFAULT_BLOCK_ROWS):
    """Masked grouped-query attention output, float64.

    q: [B, Hq, S, D]; k, v: [B, Hkv, S, D] (any real dtype, widened exactly).
    rows: optional sorted-or-not list of query positions to evaluate (all when
    None); the result then has shape [B, Hq, len(rows), D].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, Hq, rows.size, D), dtype=np.float64)
    for b in range(B):
        for a in range(Hq):
            h = kv_head(a, Hq, Hkv)
            kh = k[b, h].astype(np.float64)
            vh = v[b, h].astype(np.float64)
            for r0 in range(0, rows.size, block_rows):
                rb = rows[r0:r0 + block_rows]
                p = weights(q[b, a, rb].astype(np.float64), kh, rb, kind, window,
                            global_idx, scale)
                out[b, a, r0:r0 + rb.size] = p @ vh
    return out


def visible_pair_count(S, kind, window=0, global_idx=(), block_rows=DEFAULT_BLOCK_ROWS):
    """Number of visible (query, key) pairs of one head, by counting the mask."""
    total = 0
    for r0 in range(0, S, block_rows):
        rb = np.arange(r0, min(S, r0 + block_rows))
        total += int(visibility(rb, S, kind, window, global_idx).sum())
    return total


def effective_flops(B, Hq, S, D, kind, window=0, global_idx=()):
    """Unmasked FLOPs of the forward pass: two multiply-adds chains (QK^T and PV)
    of length D per visible pair and query head, two FLOPs per multiply-add."""
    return 4 * D * visible_pair_count(S, kind, window, global_idx) * B * Hq
