// kernel_fp32.hip -- fp32 fused attention forward (vector ALU).
//
// One workgroup = 16 query rows of one query head; sixteen lanes (one DPP
// row) share a query row, each owning D / 16 of the head width for q and the
// output accumulator, so a score is 4 or 8 fused multiply-adds per lane and a
// four-step DPP reduction inside the row (every lane of the row ends with the
// same sum).  Key/value tiles of 32 rows are staged in LDS, double-buffered:
// the next tile's global loads are issued before the current tile's
// arithmetic and written to the other buffer after it.  They are consumed
// with the online softmax: per tile the running row maximum m and
// denominator l are updated as m' = max(m, max_j s_j), l' = l * 2^(m - m') +
// sum_j 2^(s_j - m'), and the accumulator is rescaled by the same 2^(m - m')
// ("Transformer 演进与变体", section Flash Attention, online-softmax
// paragraph), with the scores in log2 units (scale * log2 e folded in).  The
// n x n scores never leave registers.  All arithmetic is fp32.
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int LPR = 16;                      // lanes per query row (one DPP row)
constexpr int BM = kF32Rows;                 // query rows per workgroup
constexpr int BN = kF32Keys;                 // keys per tile
static_assert(BM * LPR == kThreads, "one workgroup holds BM rows of LPR lanes");

// Sum over the 16 lanes of a DPP row, the same value in every lane: pairs
// (quad_perm 1,0,3,2), quads (2,3,0,1), half rows (row_half_mirror), rows
// (row_mirror).  Each step adds two equal operands in swapped order, so all
// lanes hold bitwise the same sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xf, 0xf, false);
  return x;
}

template <int D, int MASK>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp32(KParams p) {
  constexpr int DQ = D / LPR;                   // dims per lane
  constexpr int NL = BN * (D / 4) / kThreads;   // float4 of K (and of V) per thread per tile
  static_assert(NL * kThreads == BN * (D / 4), "tile split over the threads");
  __shared__ float ks[2][BN][D];
  __shared__ float vs[2][BN][D];
  __shared__ int gpos_s[kMaxGlobal];

  const Sched& s = p.s;
  const int tid = threadIdx.x;
  const int r = tid / LPR;     // row within the block
  const int part = tid % LPR;  // slice of the head width
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
  for (int e = 0; e < DQ; e += 4) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_valid) x = *(const float4*)(qp + (size_t)q_row * D + part * DQ + e);
    qv[e] = x.x;
    qv[e + 1] = x.y;
    qv[e + 2] = x.z;
    qv[e + 3] = x.w;
  }
#pragma unroll
  for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;  // log2 units
  const float c2 = p.scale * 1.4426950408889634f;

  int klo, khi;
  key_range(s, it.is_global, r0, r1, &klo, &khi);
  const int kt_lo = klo / BN, kt_hi = khi / BN;
  const int n_strip = (MASK == MASK_LOCAL_GLOBAL && !it.is_global) ? cdiv(s.n_global, BN) : 0;
  const int n_it = (kt_hi - kt_lo + 1) + n_strip;

  // K and V rows of tile iter into registers (zero rows beyond S / beyond the
  // global list): float4 n of this thread is row f / (D / 4), column f % (D / 4)
  float4 kr[NL], vr[NL];
  auto fetch = [&](int iter) {
    const bool strip = iter < n_strip;
    const int kt = kt_lo + iter - n_strip;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int f = tid + n * kThreads;
      const int key = f / (D / 4), c4 = f % (D / 4);
      int row;
      if (strip) {
        const int slot = iter * BN + key;
        row = slot < s.n_global ? gpos_s[slot] : -1;
      } else {
        row = kt * BN + key;
        if (row >= s.S) row = -1;
      }
      kr[n] = make_float4(0.f, 0.f, 0.f, 0.f);
      vr[n] = kr[n];
      if (row >= 0) {
        kr[n] = *(const float4*)(kp + (size_t)row * D + c4 * 4);
        vr[n] = *(const float4*)(vp + (size_t)row * D + c4 * 4);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int f = tid + n * kThreads;
      const int key = f / (D / 4), c4 = f % (D / 4);
      *(float4*)&ks[buf][key][c4 * 4] = kr[n];
      *(float4*)&vs[buf][key][c4 * 4] = vr[n];
    }
  };

  if (n_it > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int iter = 0; iter < n_it; ++iter) {
    const int cb = iter & 1;
    if (iter + 1 < n_it) fetch(iter + 1);  // lands while this tile is computed
    const bool strip = iter < n_strip;
    const int kt = kt_lo + iter - n_strip;

    float t[BN];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; e += 4) {
        const float4 kk = *(const float4*)&ks[cb][j][part * DQ + e];
        d = fmaf(qv[e], kk.x, d);
        d = fmaf(qv[e + 1], kk.y, d);
        d = fmaf(qv[e + 2], kk.z, d);
        d = fmaf(qv[e + 3], kk.w, d);
      }
      d = row16_sum(d);
      bool vis;
      if (strip) {
        const int slot = iter * BN + j;
        if (slot < s.n_global) {
          const int g = gpos_s[slot];
          const int dist = q_row - g;
          vis = dist > s.window || -dist > s.window;  // outside the band: not yet counted
        } else {
          vis = false;
        }
      } else {
        const int kpos = kt * BN + j;
        vis = kpos < s.S && (it.is_global || visible_band(MASK, s.window, q_row, kpos));
      }
      t[j] = vis ? d * c2 : -INFINITY;
      tmax = fmaxf(tmax, t[j]);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pj = __builtin_amdgcn_exp2f(t[j] - m_use);
      l += pj;
#pragma unroll
      for (int e = 0; e < DQ; e += 4) {
        const float4 vv = *(const float4*)&vs[cb][j][part * DQ + e];
        acc[e] = fmaf(pj, vv.x, acc[e]);
        acc[e + 1] = fmaf(pj, vv.y, acc[e + 1]);
        acc[e + 2] = fmaf(pj, vv.z, acc[e + 2]);
        acc[e + 3] = fmaf(pj, vv.w, acc[e + 3]);
      }
    }
    m = m_new;
    if (iter + 1 < n_it) stash(cb ^ 1);  // the other buffer was last read before the previous barrier
    __syncthreads();
  }

  bool store = row_valid;
  if (MASK == MASK_LOCAL_GLOBAL && !it.is_global && store) {
    for (int g = 0; g < s.n_global; ++g) store = store && (gpos_s[g] != q_row);
  }
  if (store) {
    const float inv = 1.f / l;
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
