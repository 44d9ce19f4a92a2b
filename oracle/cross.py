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
    local_global   |p_i - j| <= w, or p_i is a global position, or j is one
                   ("Transformer 演进与变体", section 稀疏注意力, the Longformer
                   paragraph: a sliding window plus global tokens that see
                   and are seen by every position).  Reading: the global
                   indices are key positions (sequence positions), the same
                   for every sequence of the batch; a sequence holding fewer
                   keys has no global token at or past its end.

A query that sees no key (p_i < 0, which needs Skv < Sq) has output zero.
With Sq == Skv this is the square attention of reference.py.

Optional parts of the same call:

* ALiBi -- "Transformer 演进与变体", section 线性偏置注意力; "Trasformer 浅析",
  section 加性偏置：ALiBi; "Transformer 架构及其变体", section
  位置信息通过查询和键进入注意力: query head a adds minus its slope m_a times
  the distance between query and key to each scaled score, before the
  softmax.  Readings: the slope is indexed by the QUERY head a (the third
  page's notation), the distance is |p_i - j| (the first page's absolute form;
  it equals p_i - j on every key a causal or causal-window query sees), and
  the bias is added after the 1/sqrt(d) scaling, not scaled itself.  Slopes
  are inputs (the pages fix none; any real value is accepted).
* Distance bias -- "Trasformer 浅析", the closing section on the unified view
  (sequence attention, positional biases and graph attention as one formula):
  the logit is the scaled score plus a term b_ij, and what distinguishes the
  priors is where b_ij comes from (position, distance or graph structure).
  Reading for the distance case: b_ij is a function f_a of the signed
  distance d = j - p_i (key position minus query position), one function
  per query head, given as a table over every distance a call can produce:
  row a holds Sq + Skv - 1 values and entry d + Skv - 1 is f_a(d), for
  d in [-(Skv - 1), Sq - 1] (the table's length and offset come from the
  call's Sq and Skv, also in padded batches, where each sequence uses the
  distances of its own positions).  The term is added after the scaling and
  is not scaled itself.  ALiBi is the table -m_a |d|.
* Padded (ragged) batches -- "Trasformer 浅析", section 填充掩码与因果掩码:
  short sequences of a batch are padded and the padded positions are masked
  out.  Reading: sequence b holds q_len[b] valid query rows and kv_len[b]
  valid keys, both at the START of its rows (right padding); the call on
  sequence b is the call above with Sq = q_len[b] and Skv = kv_len[b], so
  query i sits at p_i = i + kv_len[b] - q_len[b]; padded keys are never
  visible and padded query rows are written as zero.  What the padded
  positions hold never reaches a valid output.

Layout: q [B][Hq][Sq][D], k and v [B][Hkv][Skv][D] (logical layout; strided
device layouts are a matter of the tests).  float64 on the exact inputs.

Pinned by tests/test_oracle_cross.py (ALiBi, the distance bias and padded
batches included).
"""
from __future__ import annotations

import numpy as np

FULL = "full"
CAUSAL = "causal"
CAUSAL_WINDOW = "causal_window"
LOCAL_GLOBAL = "local_global"
CROSS_MASK_KINDS = (FULL, CAUSAL, CAUSAL_WINDOW, LOCAL_GLOBAL)


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


def cross_visible_keys(Sq, Skv, i, kind, window=0, global_idx=()):
    """Visible key positions of query i, ascending (an int64 array)."""
    if kind != LOCAL_GLOBAL:
        lo, hi = cross_visible_range(Sq, Skv, i, kind, window)
        return np.arange(lo, max(lo, hi), dtype=np.int64)
    if window < 0:
        raise ValueError("local_global needs window >= 0")
    p = i + Skv - Sq
    g = sorted({int(x) for x in global_idx if 0 <= int(x) < Skv})
    if p in g:
        return np.arange(Skv, dtype=np.int64)
    band = set(range(max(0, p - window), min(Skv, p + window + 1)))
    return np.array(sorted(band | set(g)), dtype=np.int64)


def alibi_penalty(slope, p, j):
    """What ALiBi subtracts from the scaled score of query position p and key
    positions j: the head's slope times their distance."""
    return slope * np.abs(p - np.asarray(j, dtype=np.float64))


def head_slope(slopes, a, G):
    """ALiBi slope of query head a (G query heads per key/value head)."""
    return slopes[a]


def head_bias_row(table, a, G):
    """Distance-bias table row of query head a (G query heads per key/value
    head)."""
    return table[a]


def distance_bias(row, p, j, Skv):
    """The distance-bias term of query position p and key positions j: entry
    (j - p) + Skv - 1 of the head's table row (Skv: the call's key count)."""
    return np.asarray(row, dtype=np.float64)[np.asarray(j, dtype=np.int64) - p + Skv - 1]


def sequence_lengths(Sq, Skv, q_len, kv_len, b):
    """Valid query rows and keys of sequence b."""
    sq_b = Sq if q_len is None else int(q_len[b])
    skv_b = Skv if kv_len is None else int(kv_len[b])
    if not (0 <= sq_b <= Sq and 0 <= skv_b <= Skv):
        raise ValueError("lengths must lie in [0, Sq] and [0, Skv]")
    return sq_b, skv_b


def cross_attention(q, k, v, kind, window=0, scale=None, rows=None, alibi_slopes=None,
                    q_len=None, kv_len=None, global_idx=(), dist_bias=None):
    """Attention output, float64, shape [B, Hq, Sq, D]; with `rows` (query row
    indices) only those rows, shape [B, Hq, len(rows), D].  `alibi_slopes`: Hq
    slopes (None: no bias); `q_len`, `kv_len`: B valid lengths each (None: all
    Sq / Skv rows valid); `global_idx`: the global key positions of
    "local_global"; `dist_bias`: the [Hq][Sq + Skv - 1] distance-bias table
    (None: no such term)."""
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
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float64)
    if slopes is not None and slopes.shape != (Hq,):
        raise ValueError("alibi_slopes needs one slope per query head")
    table = None if dist_bias is None else np.asarray(dist_bias, dtype=np.float64)
    if table is not None and table.shape != (Hq, Sq + Skv - 1):
        raise ValueError("dist_bias needs Hq rows of Sq + Skv - 1 values")
    out = np.zeros((B, Hq, len(rows), D), dtype=np.float64)
    for b in range(B):
        sq_b, skv_b = sequence_lengths(Sq, Skv, q_len, kv_len, b)
        for a in range(Hq):
            h = a // G
            for r, i in enumerate(rows):
                if i >= sq_b:
                    continue  # padded query row
                js = cross_visible_keys(sq_b, skv_b, i, kind, window, global_idx)
                if js.size == 0:
                    continue
                kk = k[b, h, js].astype(np.float64)
                vv = v[b, h, js].astype(np.float64)
                s = float(scale) * (kk @ q[b, a, i].astype(np.float64))
                if slopes is not None:
                    s = s - alibi_penalty(head_slope(slopes, a, G), i + skv_b - sq_b, js)
                if table is not None:
                    s = s + distance_bias(head_bias_row(table, a, G), i + skv_b - sq_b, js, Skv)
                e = np.exp(s - s.max())
                out[b, a, r] = (e / e.sum()) @ vv
    return out


def cross_visible_pairs(Sq, Skv, kind, window=0, global_idx=()):
    """Visible (query, key) pairs of one head."""
    tot = 0
    for i in range(Sq):
        tot += cross_visible_keys(Sq, Skv, i, kind, window, global_idx).size
    return tot
