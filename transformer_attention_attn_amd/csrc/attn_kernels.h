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
  float bias_k;          // ALiBi slope or distance bias -> score units: 1 / |scale|,
                         // or log2(e) for scale 0
  const float* bias;     // device [Hq][bias_len] distance-bias table, or null: entry
                         // d + Skv - 1 of row a is added to query head a's logits at
                         // signed distance d = key position - query position
  int bias_len;          // Sq + Skv - 1
  const unsigned* layout;  // device block-sparse layout (64-position blocks), or null
  int lay_nw;              // words per layout row
};

// Longest sequence of a block-sparse call (its tile list lives in registers,
// 64 tiles per register), and the longest the short-list kernels take.
constexpr int kSparseMaxKeys = 32768;
constexpr int kSparseShortKeys = 8192;

// Workgroup shapes used by the two kernels.
constexpr int kF32Rows = 16;   // query rows per fp32 work item (one head, 16 lanes per row)
constexpr int kF32Keys = 32;   // keys per fp32 tile
constexpr int kBf16Rows = 32 * kBf16Waves;  // query rows per bf16 work item (heads packed)
constexpr int kBf16GlobalRows = 32;          // global rows per query head in a bf16 global item
// keys per bf16 tile: 128 at D = 128 (a 64-MFMA block), 64 at D = 64 (32 MFMAs)
ATTN_HD int bf16_keys_per_tile(int D) { return D == 128 ? 128 : 64; }

hipError_t launch_fp32(const KParams& p, int D, hipStream_t stream);
hipError_t launch_bf16_d64(const KParams& p, hipStream_t stream);   // kernel_bf16.hip, D = 64 build
hipError_t launch_bf16_d128(const KParams& p, hipStream_t stream);  // kernel_bf16.hip, D = 128 build
// persistent form of the D = 128 dense square kernel (masks FULL, CAUSAL,
// CAUSAL_WINDOW): `grid` workgroups walk the s.n_items work items
hipError_t launch_bf16_pers_d128(const KParams& p, int grid, hipStream_t stream);
// FP8 inputs, bf16 output, D = 64 or 128, every mask (e5m2: q, k, v in E5M2
// instead of E4M3)
hipError_t launch_fp8(const KParams& p, int D, bool e5m2, hipStream_t stream);  // kernel_fp8.hip

}  // namespace attn
