"""fp64 CPU oracle for decode attention against a key/value cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP path, and none with the full-sequence oracle in
reference.py either (the tests compare the two).

What it computes (plain definition, one query row at a time):

* Decode step -- "Trasformer 浅析", section 推理：KV 缓存: the output of the
  query at step t is the softmax of its scaled scores against the cached keys
  of positions 1..t, applied to the cached values of the same positions.
* Prefill and decode -- "Transformer 架构及其变体", section
  预填充创建缓存，解码复用缓存: each decode step appends the new position's
  key and value to the cache and lets the new query read the stored history;
  the sequences of a batch may hold caches of different lengths S_r.
* Heads -- as in the full-sequence oracle: query head a reads key/value head
  floor(a / (Hq / Hkv)) ("Transformer 架构及其变体", section
  带显式形状的因果自注意力; all query heads of a group read one cache,
  "第 8 章 AI 算法Transformer大模型", section 8.2.1 KV 缓存的内存瓶颈).

Readings taken where the pages leave a step open:

* Several new positions per step (Sq >= 1, e.g. a chunk of a prompt or a few
  draft tokens): they are the last Sq positions of the cache, query i at
  position L - Sq + i, already appended.  "causal" lets query i see cache
  positions 0 .. L - Sq + i; "full" lets every query see all L positions.
  With Sq = 1 the two coincide and equal the page's decode formula.
* Sliding window in decode ("causal_window", window w >= 1) -- "Transformer
  演进与变体", section 稀疏注意力 (Mistral's window of 4096): query i at
  position p = L - Sq + i sees the cache positions j with p - w < j <= p,
  the same visibility as the full-sequence oracle's causal_window mask, so
  only the last w positions are read.
* A query that sees no position (L - Sq + i < 0, or L = 0) has output zero.
* Cache positions at or beyond a sequence's length L are not part of the
  sequence: whatever they hold (even NaN) never reaches the output.

Layout: q is [B][Hq][Sq][D]; the caches are [B][Hkv][Smax][D] with L_b <= Smax
valid positions for sequence b.  All arithmetic is float64 on the exact input
values.

Pinned by tests/test_oracle_decode.py (the full-sequence oracle's last rows,
also under the window; padding that must not leak; closed forms, a window of
one position among them; a grouped-head reduction and a pure-Python loop).
"""
from __future__ import annotations

import numpy as np

FULL = "full"
CAUSAL = "causal"
CAUSAL_WINDOW = "causal_window"
DECODE_MASK_KINDS = (FULL, CAUSAL, CAUSAL_WINDOW)


def decode_visible_range(L, Sq, i, kind, window=0):
    """Cache positions [lo, hi) that query i (of Sq new ones, at position
    L - Sq + i) sees in a cache of L positions (lo == hi: none)."""
    if kind == FULL:
        return 0, L
    p = L - Sq + i
    if kind == CAUSAL:
        return 0, max(0, min(L, p + 1))
    if kind == CAUSAL_WINDOW:
        if window < 1:
            raise ValueError("causal_window needs window >= 1")
        hi = max(0, min(L, p + 1))
        return min(hi, max(0, p - window + 1)), hi
    raise ValueError(f"unknown decode mask kind {kind!r}")


def decode_visible_count(L, Sq, i, kind, window=0):
    """Number of cache positions query i (of Sq new ones) sees in a cache of L."""
    lo, hi = decode_visible_range(L, Sq, i, kind, window)
    return hi - lo


def decode_attention(q, k_cache, v_cache, kind, cache_len=None, scale=None, window=0):
    """Decode attention output, float64, shape [B, Hq, Sq, D].

    q: [B, Hq, Sq, D]; k_cache, v_cache: [B, Hkv, Smax, D]; cache_len: B ints in
    [0, Smax] (all Smax when None); window: the w of "causal_window".
    """
    q = np.asarray(q)
    kc = np.asarray(k_cache)
    vc = np.asarray(v_cache)
    B, Hq, Sq, D = q.shape
    Hkv, Smax = kc.shape[1], kc.shape[2]
    if kc.shape != (B, Hkv, Smax, D) or vc.shape != kc.shape:
        raise ValueError("shape mismatch between q and the caches")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    lens = [Smax] * B if cache_len is None else [int(x) for x in cache_len]
    if len(lens) != B or any(x < 0 or x > Smax for x in lens):
        raise ValueError("cache_len must hold B lengths in [0, Smax]")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    for b in range(B):
        for a in range(Hq):
            h = a // G
            for i in range(Sq):
                lo, hi = decode_visible_range(lens[b], Sq, i, kind, window)
                if hi == lo:
                    continue
                keys = kc[b, h, lo:hi].astype(np.float64)
                vals = vc[b, h, lo:hi].astype(np.float64)
                s = float(scale) * (keys @ q[b, a, i].astype(np.float64))
                e = np.exp(s - s.max())
                out[b, a, i] = (e / e.sum()) @ vals
    return out


def decode_cache_bytes(B, Hkv, D, cache_len, elem_bytes, Sq=1, kind=CAUSAL, window=0):
    """Bytes of the key and value cache entries that one call must read: 2 *
    Hkv * D * elem_bytes per cached position that some query sees, summed over
    the sequences (the per-layer payload of "Transformer 架构及其变体", section
    预填充创建缓存，解码复用缓存; under a window, the last window + Sq - 1
    positions at most)."""
    n = 0
    for L in cache_len:
        los, his = zip(*(decode_visible_range(int(L), Sq, i, kind, window) for i in range(Sq)))
        lo, hi = min(los), max(his)
        n += max(0, hi - lo)
    return 2 * Hkv * D * elem_bytes * n


def decode_effective_flops(Hq, Sq, D, cache_len, kind, window=0):
    """Two multiply-add chains of length D per visible (query, cache position)
    pair and query head, two FLOPs per multiply-add."""
    pairs = 0
    for L in cache_len:
        for i in range(Sq):
            pairs += decode_visible_count(int(L), Sq, i, kind, window)
    return 4 * D * pairs * Hq
