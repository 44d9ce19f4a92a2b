// kernel_bf16.hip -- bf16 fused attention forward on gfx950 matrix cores.
//
// Method: exact tiled attention with the online softmax ("Transformer 演进与变
// 体", section Flash Attention: tiling, online softmax, kernel fusion): the
// query rows stay in registers, key/value tiles stream through LDS, and per
// tile the running row maximum m and denominator l are updated as
//   m' = max(m, max_j s_j),  l' = l * 2^(m - m') + sum_j 2^(s_j - m'),
// with the output accumulator rescaled by 2^(m - m').  Scores are kept in log2
// units (s = q.k * scale * log2(e)), so exp becomes one v_exp_f32.  Only O is
// written to HBM.
//
// gfx950 mapping (one workgroup = four wave64, 32 query rows per wave):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q^T
//     from registers.  In the 32x32 accumulator each lane owns one query
//     (lane % 32) and 16 of the 32 keys, so the row max and row sum are mostly
//     in-lane; one v_permlane32_swap joins the two lane halves.
//   * O^T += V^T P^T on the same instruction: B = P^T straight from the score
//     registers (converted to bf16, round to nearest even), A = V^T from a
//     transposed LDS tile.  The accumulator lane again owns one query, so the
//     rescale factor is a per-lane scalar.
//   * K and V tiles (16 KiB each) are double-buffered in LDS; the next tile's
//     global loads are issued before the current tile's matrix work and land
//     in LDS after it, so HBM latency hides behind the MFMAs.
//   * Query heads that share a key/value head are packed into one workgroup
//     (up to four, one per wave), so each K/V tile is staged once per group.
//   * Fully masked tiles are never visited (mask-aware key-tile ranges), and
//     a wave skips the matrix work of tiles that are empty for its own rows;
//     only partial tiles evaluate the per-element mask.
#include "attn_kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max of x over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

template <int D, int MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(KParams p) {
  constexpr int BN = 8192 / D;          // keys per tile (16 KiB of K)
  constexpr int NKB = BN / 32;          // 32-key blocks of S^T
  constexpr int NDC = D / 16;           // reduction steps of S^T (16 dims each)
  constexpr int NDB = D / 32;           // 32-dim blocks of O^T
  constexpr int NPC = BN / 16;          // reduction steps of O^T (16 keys each)
  constexpr int KCH = D / 8;            // 16-byte chunks per K row
  constexpr int KSTRIDE = D * 2 + 16;   // padded K row in LDS: rows r..r+7 hit distinct banks
  constexpr int KTILE = BN * KSTRIDE;
  constexpr int VTILE = BN * D * 2;
  constexpr int BUF = KTILE + VTILE;
  constexpr int KLOADS = BN * KCH / kThreads;  // 16-byte K chunks per thread per tile
  static_assert(KLOADS * kThreads == BN * KCH, "K tile split");
  static_assert((BN / 8) * (D / 4) == kThreads, "V tile split: 8 keys x 4 dims per thread");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];
  __shared__ int gpos_s[kMaxGlobal];

  const Sched& s = p.s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // lane half: selects the k sub-range of an MFMA operand
  const Item it = decode_item(s, blockIdx.x);

  if (MASK == MASK_LOCAL_GLOBAL) {
    if (tid < kMaxGlobal) gpos_s[tid] = tid < s.n_global ? p.gpos[tid] : 0;
    __syncthreads();
  }

  // ---- rows of this wave -------------------------------------------------
  const int wph = 4 / s.HP;                       // waves per query head
  const int a = it.kvh * s.G + it.hg * s.HP + wave / wph;
  const int rpart = wave % wph;
  int q_row, wqa = 0, wqb = -1, r0 = 0, r1 = 0;
  bool row_valid;
  if (!it.is_global) {
    r0 = it.blk * s.BMh;
    r1 = imin(r0 + s.BMh, s.S) - 1;
    const int q0 = r0 + rpart * 32;
    q_row = q0 + l32;
    row_valid = q_row < s.S;
    wqa = q0;
    wqb = imin(q0 + 31, s.S - 1);
  } else {
    const int slot = it.blk * s.BMh + rpart * 32 + l32;
    row_valid = slot < s.n_global;
    q_row = row_valid ? gpos_s[slot] : 0;
    const int first = it.blk * s.BMh + rpart * 32;
    wqa = 0;
    wqb = first < s.n_global ? 0 : -1;  // wave active iff it holds a global row
  }
  const bool wave_active = wqa <= wqb;

  const size_t S = (size_t)s.S;
  const __bf16* qp = (const __bf16*)p.q + (size_t)(it.b * s.Hq + a) * S * D;
  const __bf16* kp = (const __bf16*)p.k + (size_t)(it.b * s.Hkv + it.kvh) * S * D;
  const __bf16* vp = (const __bf16*)p.v + (size_t)(it.b * s.Hkv + it.kvh) * S * D;

  // ---- Q^T operand: lane holds query q_row, dims 16*dc + 8*hf + [0, 8) -----
  bf16x8 qf[NDC];
  {
    const u32x4 flip = (p.qmode == 1) ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                                      : u32x4{0u, 0u, 0u, 0u};
    const bool zero = (p.qmode == 2) || !row_valid;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (!zero) x = *(const u32x4*)(qp + (size_t)q_row * D + dc * 16 + hf * 8);
      x ^= flip;
      qf[dc] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- key tiles to visit ------------------------------------------------
  int klo, khi;
  key_range(s, it.is_global, r0, r1, &klo, &khi);
  const int kt_lo = klo / BN, kt_hi = khi / BN;
  const int has_strip = (MASK == MASK_LOCAL_GLOBAL && !it.is_global && s.n_global > 0) ? 1 : 0;
  const int n_it = (kt_hi - kt_lo + 1) + has_strip;

  // Loader assignment.  K: 16-byte chunk f = n*256 + tid of the tile, i.e. key
  // f / KCH, chunk f % KCH (16 consecutive lanes read one row), byte offset
  // f * 16 within the tile.  V: thread owns 8 keys x 4 dims: key group
  // vg = tid / (D/4) -> (c, h) = (vg >> 1, vg & 1), keys 16c + 4h + {0..3} and
  // 16c + 8 + 4h + {0..3} (the key order of the P^T operand), dims
  // 4 * (tid % (D/4)) + [0, 4).
  const int vg = tid / (D / 4);
  const int vdg = tid % (D / 4);
  const int vc = vg >> 1, vh = vg & 1;
  const int v_off = (16 * vc + 4 * vh) * D * 2 + vdg * 8;  // + key step (t&3) + 8 (t>>2) rows

  u32x4 kreg[KLOADS];
  u32x2 vreg[8];

  // Band tile kt through raw buffer loads: the descriptor covers only the
  // rows [kt*BN, min(S, kt*BN + BN)), so rows past the end read as zero and no
  // per-lane address arithmetic or branch is needed.
  auto load_band = [&](int kt) {
    const int row0 = kt * BN;
    const int nbytes = imin(BN, s.S - row0) * D * 2;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kp + (size_t)row0 * D), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vp + (size_t)row0 * D), (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int n = 0; n < KLOADS; ++n)
      kreg[n] = __builtin_amdgcn_raw_buffer_load_b128(kr, tid * 16, n * kThreads * 16, 0);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      vreg[t] = __builtin_amdgcn_raw_buffer_load_b64(vr, v_off + ((t & 3) + 8 * (t >> 2)) * D * 2, 0, 0);
  };

  // Strip tile: the global tokens' rows, gathered; slots past n_global repeat
  // a valid row (their scores are masked, so they carry zero weight).
  auto load_strip = [&]() {
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int f = n * kThreads + tid;
      const int key = f / KCH, ch = f % KCH;
      const int row = gpos_s[imin(key, s.n_global - 1)];
      kreg[n] = *(const u32x4*)(kp + (size_t)row * D + ch * 8);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int key = 16 * vc + 4 * vh + (t & 3) + 8 * (t >> 2);
      const int row = gpos_s[imin(key, s.n_global - 1)];
      vreg[t] = *(const u32x2*)(vp + (size_t)row * D + vdg * 4);
    }
  };

  auto store_tile = [&](int buf) {
    unsigned char* kb = smem + buf * BUF;
    unsigned char* vb = kb + KTILE;
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int f = n * kThreads + tid;
      const int key = f / KCH, ch = f % KCH;
      *(u32x4*)(kb + key * KSTRIDE + ch * 16) = kreg[n];
    }
    // transpose 8 keys x 4 dims into 4 slots of 8 keys (one per dim)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x4 w;
      w.x = __builtin_amdgcn_perm(vreg[1][j >> 1], vreg[0][j >> 1], sel);
      w.y = __builtin_amdgcn_perm(vreg[3][j >> 1], vreg[2][j >> 1], sel);
      w.z = __builtin_amdgcn_perm(vreg[5][j >> 1], vreg[4][j >> 1], sel);
      w.w = __builtin_amdgcn_perm(vreg[7][j >> 1], vreg[6][j >> 1], sel);
      const int d = vdg * 4 + j;
      const int phys = d ^ ((d >> 3) & 3);  // bank-conflict-free for both writes and reads
      *(u32x4*)(vb + ((vc * 2 + vh) * D + phys) * 16) = w;
    }
  };

  // ---- accumulators --------------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // m_run: the reference maximum (in units of q.k) the weights of query q_row
  // are exponentiated against.  It is raised only when a tile's maximum
  // exceeds it by more than 2^kLazy in weight, so the output rescale is rare;
  // weights are then at most 2^kLazy, far inside fp32 and bf16 range, and
  // O / l is unchanged (numerator and denominator share the reference).
  constexpr float kLazy = 8.f;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share of the denominator (its 16 of each 32 keys)
  const float c = p.c;
  const int lswz = l32 ^ ((l32 >> 3) & 3);  // V^T read slot within a 32-dim block
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  if (has_strip) load_strip(); else load_band(kt_lo);
  store_tile(0);

  for (int iter = 0; iter < n_it; ++iter) {
    __syncthreads();  // tile iter is in LDS; buffer (iter+1)&1 is free
    const bool more = iter + 1 < n_it;
    const int kt = kt_lo + iter - has_strip;
    if (more) load_band(kt + 1);

    const int buf = iter & 1;
    const unsigned char* kb = smem + buf * BUF;
    const unsigned char* vb = kb + KTILE;
    const bool strip = has_strip && iter == 0;

    int cls;
    if (!wave_active) cls = TILE_EMPTY;
    else if (strip) cls = TILE_PARTIAL;
    else if (it.is_global) cls = (kt * BN + BN > s.S) ? TILE_PARTIAL : TILE_FULL;
    else cls = classify_tile(MASK, s.window, s.S, wqa, wqb, kt * BN, BN);

    if (cls != TILE_EMPTY) {
      // S^T = K Q^T
      f32x16 sacc[NKB];
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kbk][r] = 0.f;
        const unsigned char* krow = kb + (kbk * 32 + l32) * KSTRIDE + hf * 16;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          const bf16x8 ka = *(const bf16x8*)(krow + dc * 32);
          sacc[kbk] = mfma32(ka, qf[dc], sacc[kbk]);
        }
      }
      // per-element mask on partial tiles; register r of block kbk holds key
      // 32*kbk + 8*(r/4) + 4*hf + r%4 of the tile for query q_row
      if (cls == TILE_PARTIAL) {
        asm volatile("");  // keep this a branch: full tiles skip it
        if (MASK == MASK_LOCAL_GLOBAL && strip) {
#pragma unroll
          for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbk * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
              const int dist = q_row - gpos_s[key < kMaxGlobal ? key : 0];
              const bool vis = key < s.n_global && (dist > s.window || -dist > s.window);
              sacc[kbk][r] = vis ? sacc[kbk][r] : -INFINITY;
            }
        } else {
          // visible keys of this lane's query as an interval of tile-relative
          // indices, shifted by the lane half so each test is against an
          // immediate: lo <= 32*kbk + 8*(r/4) + r%4 <= hi
          long long lo, hi;
          if (it.is_global) { lo = 0; hi = (long long)s.S - 1; }
          else row_interval(MASK, s.window, s.S, q_row, &lo, &hi);
          const long long base = (long long)kt * BN + 4 * hf;
          const long long tail = (long long)s.S - 1;
          const int lo_r = (int)(lo - base < -1 ? -1 : (lo - base > BN ? BN : lo - base));
          const long long hi_a = hi < tail ? hi : tail;
          const int hi_r = (int)(hi_a - base < -1 ? -1 : (hi_a - base > BN ? BN : hi_a - base));
#pragma unroll
          for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbk * 32 + 8 * (r >> 2) + (r & 3);
              const bool vis = key >= lo_r && key <= hi_r;
              sacc[kbk][r] = vis ? sacc[kbk][r] : -INFINITY;
            }
        }
      }
      // online softmax (scores in units of q.k; c = |scale| log2 e)
      float mx = -INFINITY;
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kbk][r]);
      mx = pair_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx * c > m_run * c + kLazy)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
      bf16x8 pb[NPC];
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int t = 0; t < 8; t += 2) {
            bf16x2 pr;
            pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kbk][half * 8 + t], c, -mc));
            pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kbk][half * 8 + t + 1], c, -mc));
            // the denominator sums exactly the rounded weights used in P.V
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
            pb[kbk * 2 + half][t] = pr[0];
            pb[kbk * 2 + half][t + 1] = pr[1];
          }
        }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int pc = 0; pc < NPC; ++pc) {
          const bf16x8 va = *(const bf16x8*)(vb + ((pc * 2 + hf) * D + db * 32 + lswz) * 16);
          oacc[db] = mfma32(va, pb[pc], oacc[db]);
        }
    }

    if (more) store_tile((iter + 1) & 1);
  }

  // ---- epilogue: O = O^T / l, round to bf16, store --------------------------
  {
    const unsigned lu = __float_as_uint(l_run);
    const float l_other = __uint_as_float(__shfl_xor((int)lu, 32));
    const float l_tot = l_run + l_other;
    bool store = row_valid && wave_active;
    if (MASK == MASK_LOCAL_GLOBAL && !it.is_global && store) {
      for (int g = 0; g < s.n_global; ++g) store = store && (gpos_s[g] != q_row);
    }
    if (store) {
      const float inv = 1.f / l_tot;
      __bf16* op = (__bf16*)p.o + ((size_t)(it.b * s.Hq + a) * S + q_row) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = (__bf16)(oacc[db][g4 * 4 + t] * inv);
          *(bf16x4*)(op + db * 32 + g4 * 8 + hf * 4) = w;
        }
    }
  }
}

template <int D>
hipError_t launch_d(const KParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.s.n_items), block(kThreads);
  switch (p.s.mask) {
    case MASK_FULL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_FULL>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL_WINDOW: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL_WINDOW>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_LOCAL_GLOBAL>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16(const KParams& p, int D, hipStream_t stream) {
  return D == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace attn
