// attn_sched.h -- mask-aware work decomposition shared by the host planner and the
// kernels (host+device inline functions, no state).
//
// A work item is one workgroup: (batch b, key/value head h, group of query
// heads of h, block of query rows).  Each item walks only the key tiles that
// its rows can see, so fully masked tiles are never touched (the saving the
// sliding-window and Longformer paragraphs of "Transformer 演进与变体",
// section 稀疏注意力, describe: work proportional to the visible pairs).
//
// For the local+global mask the pattern is split in three parts:
//   * band items: rows of one block, key tiles covering |i - j| <= w;
//   * one extra "strip" tile per band item holding the global tokens' keys
//     (columns j in G outside the band of row i);
//   * global items: the rows i in G, gathered (GR per query head per item),
//     each seeing all S keys.
// Band items compute global rows too but never store them; the global items
// own those rows.
#pragma once

#ifdef __HIPCC__
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attn {

enum { MASK_FULL = 0, MASK_CAUSAL = 1, MASK_CAUSAL_WINDOW = 2, MASK_LOCAL_GLOBAL = 3 };
enum { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

struct Sched {
  int B, Hq, Hkv, S;
  int G;        // query heads per key/value head
  int HP;       // query heads packed in one work item
  int NHG;      // G / HP head groups per key/value head
  int BMh;      // query rows per head per work item
  int BN;       // keys per tile
  int T;        // row blocks per head: ceil(S / BMh)
  int GR;       // global rows per query head in a global item
  int P;        // B * Hkv * NHG (item "pairs")
  int mask, window, n_global;
  int n_gblocks;           // global-row blocks per pair: ceil(n_global / GR) (local+global only)
  long long n_global_items;  // P * n_gblocks, numbered first
  long long n_items;         // total workgroups
  // attn_fwd_ex: Sk keys (S is then the number of query rows); query row i
  // sits at key position i + off.  attn_fwd: Sk = S, off = 0.
  int Sk, off;
};

struct Item {
  int b, kvh, hg;     // batch, key/value head, head group
  int is_global;      // 1: rows are global tokens (gathered)
  int blk;            // row block (band items) or global-row block (global items)
};

ATTN_HD int cdiv(int a, int b) { return (a + b - 1) / b; }
ATTN_HD int imin(int a, int b) { return a < b ? a : b; }
ATTN_HD int imax(int a, int b) { return a > b ? a : b; }

// Heads packed per work item: the largest of {8, 4, 2, 1} dividing G.  Packing the
// query heads of one key/value head into one workgroup lets every staged K/V
// tile serve all of them ("Transformer 演进与变体", section GQA：分组查询注意力:
// a group of query heads shares one key/value head).
ATTN_HD int heads_per_item(int G) {
  return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

ATTN_HD Sched make_sched(int B, int Hq, int Hkv, int S, int mask, int window, int n_global,
                         int rows_per_wg, int BN, int pack_heads, int global_rows) {
  Sched s;
  s.B = B; s.Hq = Hq; s.Hkv = Hkv; s.S = S;
  s.G = Hq / Hkv;
  s.HP = pack_heads ? heads_per_item(s.G) : 1;
  s.NHG = s.G / s.HP;
  s.BMh = rows_per_wg / s.HP;
  s.BN = BN;
  s.T = cdiv(S, s.BMh);
  s.P = B * Hkv * s.NHG;
  s.mask = mask; s.window = window;
  s.n_global = (mask == MASK_LOCAL_GLOBAL) ? n_global : 0;
  s.GR = global_rows;
  s.n_gblocks = s.n_global > 0 ? cdiv(s.n_global, s.GR) : 0;
  s.n_global_items = (long long)s.P * s.n_gblocks;
  s.n_items = s.n_global_items + (long long)s.P * s.T;
  s.Sk = S;
  s.off = 0;
  return s;
}

// Item numbering: global-row items first (each spans all S keys, the longest),
// then band items.  Within band items, consecutive ids walk the pairs
// fastest, so that when P is a multiple of 8 every item of one pair lands on
// the same XCD (workgroups are dealt to the 8 XCDs round-robin by id) and the
// pair's K/V stays in that XCD's L2.  Causal masks visit row blocks from the
// last (most key tiles) to the first, so the longest items start first.
ATTN_HD Item decode_item(const Sched& s, int id) {
  // 32-bit arithmetic: the host rejects launches with more than 2^31 - 1 items
  Item it;
  int pair, rank;
  const int ngi = (int)s.n_global_items;
  if (id < ngi) {
    it.is_global = 1;
    pair = id % s.P;
    rank = id / s.P;
    it.blk = rank;
  } else {
    it.is_global = 0;
    const int w = id - ngi;
    pair = w % s.P;
    rank = w / s.P;
    const int heavy_last = (s.mask == MASK_CAUSAL || s.mask == MASK_CAUSAL_WINDOW);
    it.blk = heavy_last ? (s.T - 1 - rank) : rank;
  }
  const int per_b = s.Hkv * s.NHG;
  it.b = pair / per_b;
  const int rem = pair % per_b;
  it.kvh = rem / s.NHG;
  it.hg = rem % s.NHG;
  return it;
}

// Range [*klo, *khi] (inclusive) of keys that rows [r0, r1] (inclusive) can see
// through the band / causal structure (globals excluded).
ATTN_HD void key_range(const Sched& s, int is_global, int r0, int r1, int* klo, int* khi) {
  int lo = 0, hi = s.S - 1;
  if (!is_global) {
    switch (s.mask) {
      case MASK_CAUSAL: hi = r1; break;
      case MASK_CAUSAL_WINDOW: lo = imax(0, r0 - s.window + 1); hi = r1; break;
      case MASK_LOCAL_GLOBAL:
        lo = imax(0, r0 - s.window);
        hi = (long long)r1 + s.window >= (long long)s.S ? s.S - 1 : r1 + s.window;
        break;
      default: break;
    }
  }
  *klo = lo; *khi = hi;
}

// Per-pair visibility, band part only (globals are handled by the strip tile
// and the global items).
ATTN_HD bool visible_band(int mask, int window, int i, int j) {
  switch (mask) {
    case MASK_CAUSAL: return j <= i;
    case MASK_CAUSAL_WINDOW: return j <= i && j > i - window;
    case MASK_LOCAL_GLOBAL: { int d = i - j; return d <= window && -d <= window; }
    default: return true;
  }
}

// Visible keys of band row i, as an inclusive interval [*lo, *hi] of absolute
// key positions (globals excluded; the tail j < S is applied by the caller).
ATTN_HD void row_interval(int mask, int window, int S, int i, long long* lo, long long* hi) {
  switch (mask) {
    case MASK_CAUSAL: *lo = 0; *hi = i; break;
    case MASK_CAUSAL_WINDOW: *lo = (long long)i - window + 1; *hi = i; break;
    case MASK_LOCAL_GLOBAL: *lo = (long long)i - window; *hi = (long long)i + window; break;
    default: *lo = 0; *hi = (long long)S - 1; break;
  }
}

// Classify the key tile [ka, ka + BN) for query rows [qa, qb] (band rows, a
// contiguous range).  Keys at or beyond S always make the tile partial.
ATTN_HD int classify_tile(int mask, int window, int S, int qa, int qb, int ka, int BN) {
  int kb = ka + BN - 1;
  int tail = kb >= S;
  if (tail) kb = S - 1;
  int full = 0, empty = 0;
  switch (mask) {
    case MASK_CAUSAL:
      empty = ka > qb;
      full = kb <= qa;
      break;
    case MASK_CAUSAL_WINDOW:
      empty = (ka > qb) || (kb <= qa - window);
      full = (kb <= qa) && (ka > qb - window);
      break;
    case MASK_LOCAL_GLOBAL:
      empty = (ka - qb > window) || (qa - kb > window);
      full = (kb - qa <= window) && (qb - ka <= window);
      break;
    default:
      full = 1;
      break;
  }
  if (empty) return TILE_EMPTY;
  if (full && !tail) return TILE_FULL;
  return TILE_PARTIAL;
}

}  // namespace attn
