// kernel_fp32.hip -- fp32 fused attention forward (vector ALU).
//
// One workgroup = 64 query rows of one query head; four lanes share a row,
// each owning a quarter of the head width for q and the output accumulator.
// Key/value tiles of 32 rows are staged in LDS and consumed with the online
// softmax: per tile the running row maximum m and denominator l are updated
// as m' = max(m, max_j s_j), l' = l * exp(m - m') + sum_j exp(s_j - m'), and
// the accumulator is rescaled by the same exp(m - m') ("Transformer 演进与变
// 体", section Flash Attention, online-softmax paragraph).  The n x n scores
// never leave registers.  All arithmetic is fp32.
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int BM = kF32Rows;
constexpr int BN = kF32Keys;

template <int D, int MASK>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp32(KParams p) {
  constexpr int DQ = D / 4;  // dims per lane
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  __shared__ int gpos_s[kMaxGlobal];

  const Sched& s = p.s;
  const int tid = threadIdx.x;
  const int r = tid >> 2;      // row within the block
  const int part = tid & 3;    // quarter of the head width
  const Item it = decode_item(s, blockIdx.x);
  const int a = it.kvh * s.G + it.hg;  // HP == 1 for this kernel

  if (MASK == MASK_LOCAL_GLOBAL) {
    if (tid < kMaxGlobal) gpos_s[tid] = tid < s.n_global ? p.gpos[tid] : 0;
    __syncthreads();
  }

  // rows of this work item
  int q_row;
  bool row_valid;
  int r0 = 0, r1 = 0;
  if (!it.is_global) {
    r0 = it.blk * BM;
    r1 = imin(r0 + BM, s.S) - 1;
    q_row = r0 + r;
    row_valid = q_row < s.S;
  } else {
    int slot = it.blk * BM + r;
    row_valid = slot < s.n_global;
    q_row = row_valid ? gpos_s[slot] : 0;
  }

  const size_t S = (size_t)s.S;
  const float* qp = (const float*)p.q + ((size_t)(it.b * s.Hq + a) * S) * D;
  const float* kp = (const float*)p.k + ((size_t)(it.b * s.Hkv + it.kvh) * S) * D;
  const float* vp = (const float*)p.v + ((size_t)(it.b * s.Hkv + it.kvh) * S) * D;

  float qv[DQ], acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qv[e] = row_valid ? qp[(size_t)q_row * D + part * DQ + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int klo, khi;
  key_range(s, it.is_global, r0, r1, &klo, &khi);
  const int kt_lo = klo / BN, kt_hi = khi / BN;
  const int n_strip = (MASK == MASK_LOCAL_GLOBAL && !it.is_global) ? cdiv(s.n_global, BN) : 0;
  const int n_it = (kt_hi - kt_lo + 1) + n_strip;

  for (int iter = 0; iter < n_it; ++iter) {
    const bool strip = iter < n_strip;
    const int kt = kt_lo + iter - n_strip;
    // stage K and V rows of this tile (zero rows beyond S / beyond the global list)
    for (int f = tid; f < BN * (D / 4); f += kThreads) {
      int key = f / (D / 4);
      int c4 = f % (D / 4);
      int row;
      if (strip) {
        int slot = iter * BN + key;
        row = slot < s.n_global ? gpos_s[slot] : -1;
      } else {
        row = kt * BN + key;
        if (row >= s.S) row = -1;
      }
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (row >= 0) {
        kk = *(const float4*)(kp + (size_t)row * D + c4 * 4);
        vv = *(const float4*)(vp + (size_t)row * D + c4 * 4);
      }
      *(float4*)&ks[key][c4 * 4] = kk;
      *(float4*)&vs[key][c4 * 4] = vv;
    }
    __syncthreads();

    float t[BN];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) d = fmaf(qv[e], ks[j][part * DQ + e], d);
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      bool vis;
      if (strip) {
        int slot = iter * BN + j;
        if (slot < s.n_global) {
          int g = gpos_s[slot];
          int dist = q_row - g;
          vis = dist > s.window || -dist > s.window;  // outside the band: not yet counted
        } else {
          vis = false;
        }
      } else {
        int kpos = kt * BN + j;
        vis = kpos < s.S && (it.is_global || visible_band(MASK, s.window, q_row, kpos));
      }
      t[j] = vis ? d * p.scale : -INFINITY;
      tmax = fmaxf(tmax, t[j]);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float pj = expf(t[j] - m_use);
      l += pj;
#pragma unroll
      for (int e = 0; e < DQ; ++e) acc[e] = fmaf(pj, vs[j][part * DQ + e], acc[e]);
    }
    m = m_new;
    __syncthreads();
  }

  bool store = row_valid;
  if (MASK == MASK_LOCAL_GLOBAL && !it.is_global && store) {
    for (int g = 0; g < s.n_global; ++g) store = store && (gpos_s[g] != q_row);
  }
  if (store) {
    float inv = 1.f / l;
    float* op = (float*)p.o + ((size_t)(it.b * s.Hq + a) * S + q_row) * D + part * DQ;
#pragma unroll
    for (int e = 0; e < DQ; e += 4)
      *(float4*)(op + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv,
                                       acc[e + 3] * inv);
  }
}

template <int D>
hipError_t launch_d(const KParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.s.n_items), block(kThreads);
  switch (p.s.mask) {
    case MASK_FULL: hipLaunchKernelGGL((attn_fwd_fp32<D, MASK_FULL>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_fp32<D, MASK_CAUSAL>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL_WINDOW: hipLaunchKernelGGL((attn_fwd_fp32<D, MASK_CAUSAL_WINDOW>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((attn_fwd_fp32<D, MASK_LOCAL_GLOBAL>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp32(const KParams& p, int D, hipStream_t stream) {
  return D == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace attn
