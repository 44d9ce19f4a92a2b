// attn_decode.h -- parameters of the decode kernels (kernel_decode.hip),
// shared with the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_sched.h"

namespace attn {

// Decode attention against a key/value cache (kernel_decode.hip).  Passed by
// value as the kernel argument block.
struct DParams {
  const void* q;          // [B][Hq][Sq][D] bf16
  const void* k;          // [B][Hkv][Smax][D] bf16 cache
  const void* v;          // [B][Hkv][Smax][D] bf16 cache
  void* o;                // [B][Hq][Sq][D] bf16
  const int* cache_len;   // device, B lengths, or null (all Smax)
  float* ws;              // partial (m, l, O) slots of 32 x (D + 2) floats, or null when
                          // no (b, kvh) pair of the call can take more than one split
  int* hdr;               // cache_len given and ws set: per pair (first slot, splits),
                          // written by the pair's split 0 for the combine kernel
  int max_slots;          // partial slots the workspace holds
  int B, Hq, Hkv, Sq, Smax, G;
  int uni_splits;         // cache_len null: splits of every pair (host plan); else 0
  int causal;             // 1: query i sees positions .. L - Sq + i; 0: all L
  int window;             // 0, or w: query i sees only L - Sq + i - w < j (<= Smax)
  float c;                // |scale| * log2(e), see qmode
  int qmode;              // 0 use q, 1 use -q (negative scale), 2 use 0 (zero scale)
};
constexpr int kDecodeRows = 32;        // query rows (G * Sq) per key/value head, at most
constexpr int kDecodeWorkgroups = 256; // work items a plan may hold (one per CU)
constexpr int kDecodeMinTiles = 8;     // 32-key tiles per split, at least (one per wave)
constexpr int kDecodeTile = 32;        // keys per tile
// Splits of a key range of `tiles` tiles when a split holds at most `per`.
ATTN_HD int decode_splits(int tiles, int per) { return tiles > per ? (tiles + per - 1) / per : 1; }
// First cache position any of the Sq new queries of a sequence of L positions
// sees (window 0: no window).
ATTN_HD int decode_first_key(int L, int Sq, int window) {
  if (window == 0) return 0;
  const int lo = L - Sq - window + 1;
  return lo > 0 ? lo : 0;
}

hipError_t launch_decode(const DParams& p, int D, int grid, hipStream_t stream);

}  // namespace attn
