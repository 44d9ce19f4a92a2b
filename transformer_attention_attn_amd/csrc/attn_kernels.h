// attn_kernels.h -- parameters shared by the host dispatcher and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_sched.h"

namespace attn {

constexpr int kMaxGlobal = 64;
constexpr int kThreads = 256;  // fp32 kernel: four wave64 per workgroup
constexpr int kBf16Waves = 8;  // bf16 kernel: eight wave64 per workgroup, 32 query rows each
constexpr int kBf16Threads = 64 * kBf16Waves;

// Passed by value as the kernel argument block.
struct KParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  Sched s;
  float scale;   // fp32 kernel: the caller's scale
  float c;       // bf16 kernel: |scale| * log2(e) (> 0), see qmode
  int qmode;     // bf16 kernel: 0 use q, 1 use -q (negative scale), 2 use 0 (zero scale)
  int gpos[kMaxGlobal];  // sorted distinct global-token positions (n_global of them)
  // attn_fwd_ex only (general = 1): element strides of the batch, head and row
  // dimensions of q, k, v and o (the head dimension is contiguous)
  int general;
  long long qs[3], ks[3], vs[3], os[3];
  const int* qlen;       // device, B valid query rows per sequence, or null (all Sq)
  const int* kvlen;      // device, B valid keys per sequence, or null (all Skv)
  const float* slopes;   // device, Hq ALiBi slopes, or null (no bias)
  float alibi_k;         // slope -> score units: 1 / |scale|, or log2(e) for scale 0
  const unsigned* layout;  // device block-sparse layout (64-position blocks), or null
  int lay_nw;              // words per layout row
};

// Longest sequence of a block-sparse call (its tile list lives in registers).
constexpr int kSparseMaxKeys = 8192;

// Workgroup shapes used by the two kernels.
constexpr int kF32Rows = 64;   // query rows per fp32 work item (one head)
constexpr int kF32Keys = 32;   // keys per fp32 tile
constexpr int kBf16Rows = 32 * kBf16Waves;  // query rows per bf16 work item (heads packed)
constexpr int kBf16GlobalRows = 32;          // global rows per query head in a bf16 global item
// keys per bf16 tile: 128 at D = 128 (a 64-MFMA block), 64 at D = 64 (32 MFMAs)
ATTN_HD int bf16_keys_per_tile(int D) { return D == 128 ? 128 : 64; }

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

hipError_t launch_fp32(const KParams& p, int D, hipStream_t stream);
hipError_t launch_decode(const DParams& p, int D, int grid, hipStream_t stream);  // kernel_decode.hip
hipError_t launch_bf16_d64(const KParams& p, hipStream_t stream);   // kernel_bf16.hip, D = 64 build
hipError_t launch_bf16_d128(const KParams& p, hipStream_t stream);  // kernel_bf16.hip, D = 128 build
// persistent form of the D = 128 dense square kernel (masks FULL, CAUSAL,
// CAUSAL_WINDOW): `grid` workgroups walk the s.n_items work items
hipError_t launch_bf16_pers_d128(const KParams& p, int grid, hipStream_t stream);
// FP8 (E4M3) inputs, bf16 output, D = 128, masks without global tokens
hipError_t launch_fp8_d128(const KParams& p, hipStream_t stream);  // kernel_fp8.hip

}  // namespace attn
