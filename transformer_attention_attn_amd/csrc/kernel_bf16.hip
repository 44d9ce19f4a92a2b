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
// gfx950 mapping (one workgroup = eight wave64, 32 query rows per wave, one
// workgroup per CU: 256 query rows share every K/V tile staged in LDS):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q^T
//     from registers.  In the 32x32 accumulator each lane owns one query
//     (lane % 32) and 16 of the 32 keys, so the row max and row sum are mostly
//     in-lane; one v_permlane32_swap joins the two lane halves.
//   * O^T += V^T P^T on the same instruction: B = P^T straight from the score
//     registers (converted to bf16, round to nearest even), A = V^T from a
//     transposed LDS tile.  The accumulator lane again owns one query, so the
//     rescale factor is a per-lane scalar.
//   * Software pipeline over key tiles j: while the matrix cores compute
//     S(j+1) = K(j+1) Q^T, the vector ALUs run the softmax of S(j); while they
//     compute O += V(j) P(j), the vector ALUs finish P(j).  K and V go
//     straight from HBM into LDS (buffer/global loads with the LDS flag: no
//     staging registers) through a three-stage ring, issued two tiles ahead
//     of use, with one barrier per tile.
//     V^T operands come from row-major V tiles through ds_read_b64_tr_b16.
//     MFMA accumulation chains are interleaved (a dependent MFMA waits ~44
//     cycles, an independent one issues every 32).
//   * The output rescale runs only when a row maximum grows by more than a
//     factor 2^8 (weights stay <= 2^8, far inside bf16/fp32 range); O / l is
//     unchanged by the choice of reference maximum.
//   * Query heads that share a key/value head are packed into one workgroup
//     (up to eight), so each K/V tile is staged once per group.
//   * Fully masked tiles are never visited (mask-aware key-tile ranges); only
//     partial tiles evaluate the per-element mask.
#include "attn_kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 64;           // keys per tile
constexpr int GK = 32;           // keys per private tile of the global-row path
constexpr int NKB = BN / 32;     // 32-key blocks of S^T
static_assert(NKB == 2, "the S^T steps hold two 32-key blocks");
constexpr int NPC = BN / 16;     // 16-key reduction steps of O^T
constexpr float kLazy = 8.f;     // rescale threshold, log2 units

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max(a, b, c) in one v_max3_f32.  fmaxf would add a NaN-quieting v_max per
// operand (IEEE mode); the scores are max-reduced only to pick the reference
// maximum, so quieting is not needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max of x over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// LDS-DMA and transpose-read wrappers (plain device functions, so that the
// host pass of the template kernel sees ordinary calls)
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// 16 bytes per lane from global memory into LDS at dst + 16 * lane (dst wave-uniform)
__device__ __forceinline__ void dma16_global(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}
// same through a buffer descriptor (byte offsets voff per lane + soff uniform)
__device__ __forceinline__ void dma16_buffer(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int voff,
                                             int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, soff, 0, 0);
}
// LDS byte address of a pointer into shared memory
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One V^T operand from two transposed 8-byte reads at LDS byte addresses
// base + OFF and base + OFF + HI (see the V^T operand comment in the kernel).
// Issued as inline asm: the compiler treats the transposed-read builtin as
// possibly aliasing in-flight LDS-DMA writes and would wait for every
// outstanding global load before it, which defeats the tile prefetch.  The
// caller guarantees the tile has landed, and waits for the result with
// lds_wait_frags before any use.
template <int OFF, int HI>
__device__ __forceinline__ bf16x8 lds_tr_pair(unsigned base) {
  i16x4 lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=&v"(lo), "=&v"(hi)
               : "v"(base), "i"(OFF), "i"(OFF + HI));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The NDB V^T operands (dims 32*db + l32) of 16-key step PC of a V tile whose
// per-lane read bases are vbd[db].
template <int ROWB, int NDB, int PC>
__device__ __forceinline__ void v_frags(bf16x8 (&f)[NDB], const unsigned (&vbd)[NDB]) {
  constexpr int STEP = 16 * PC * ROWB, HI = 8 * ROWB;
#pragma unroll
  for (int db = 0; db < NDB; ++db) f[db] = lds_tr_pair<STEP, HI>(vbd[db]);
}

// Wait until at most N LDS reads are outstanding; the operands are tied to the
// wait so that no use of them is scheduled above it.
template <int N, int NDB>
__device__ __forceinline__ void lds_wait_frags(bf16x8 (&f)[NDB]) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f[0]) : "i"(N));
  asm volatile("" : "+v"(f[1]));
  if constexpr (NDB > 2) {
    asm volatile("" : "+v"(f[2]));
    asm volatile("" : "+v"(f[3]));
  }
}

// One 16-byte LDS read at LDS byte address base + OFF, as inline asm (its
// completion is waited for explicitly, like the transposed reads).
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(unsigned base) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(r) : "v"(base), "i"(OFF));
  return r;
}

// The two K operands (keys 32*kbk + l32, kbk = 0, 1) of 16-dim step DC, from
// per-lane bases kbd[DC & 3] (the swizzle repeats every four steps).
template <int ROWB, int DC>
__device__ __forceinline__ void k_frags(bf16x8 (&f)[2], const unsigned (&kbd)[4]) {
  f[0] = lds_read16<128 * (DC >> 2)>(kbd[DC & 3]);
  f[1] = lds_read16<32 * ROWB + 128 * (DC >> 2)>(kbd[DC & 3]);
}

// LDS reads issued after the K operands of step dc when the S(j+1) MFMAs of
// step dc wait for them: the operands of steps dc+1 and dc+2 (read two steps
// ahead), and the V^T operands of the first 16-key step of P.V, which are
// issued between steps NDC/2 + 1 and NDC/2 + 2.
constexpr int k_younger(int dc, int ndc, int ndb) {
  return (dc + 1 < ndc ? 2 : 0) + (dc + 2 < ndc ? 2 : 0) +
         (dc >= ndc / 2 && dc <= ndc / 2 + 1 ? 2 * ndb : 0);
}

// Steps [DC, END) of S(j+1) = K(j+1) Q^T on a three-slot ring of K operands:
// read step DC+2, wait for step DC, two MFMAs (one per 32-key block).
template <int ROWB, int NDC, int NDB, int DC, int END>
__device__ __forceinline__ void s_steps(bf16x8 (&kf)[3][2], const unsigned (&kbd)[4],
                                        const bf16x8 (&qf)[NDC], f32x16 (&sn)[2]) {
  if constexpr (DC < END) {
    if constexpr (DC + 2 < NDC) k_frags<ROWB, DC + 2>(kf[(DC + 2) % 3], kbd);
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(kf[DC % 3][0]), "+v"(kf[DC % 3][1])
                 : "i"(k_younger(DC, NDC, NDB)));
    sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[DC % 3][0], qf[DC], sn[0], 0, 0, 0);
    sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[DC % 3][1], qf[DC], sn[1], 0, 0, 0);
    s_steps<ROWB, NDC, NDB, DC + 1, END>(kf, kbd, qf, sn);
  }
}

template <int D>
struct Cfg {
  static constexpr int NDC = D / 16;            // 16-dim reduction steps of S^T
  static constexpr int NDB = D / 32;            // 32-dim blocks of O^T
  static constexpr int ROWB = D * 2;            // bytes per K or V row
  static constexpr int REG = BN * ROWB;         // bytes of one K or V tile
  static constexpr int VSH = D == 128 ? 2 : 1;  // V chunk swizzle shift
  static constexpr int BUF = 2 * REG;           // K tile then V tile
  static constexpr int NSTAGE = 3;              // LDS stages: K(j+1), K(j+2) / V(j), V(j+1) in flight
  static constexpr int NI = REG / 1024 / kBf16Waves;  // 1 KiB direct loads per wave per tile
  static_assert(NI >= 1 && NI * kBf16Waves * 1024 == REG, "tile split into 1 KiB wave loads");
  static_assert(NSTAGE * BUF <= 160 * 1024, "LDS budget of one CU");
};

template <int D, int MASK>
__global__ __launch_bounds__(kBf16Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(KParams p) {
  using C = Cfg<D>;
  constexpr int NDC = C::NDC, NDB = C::NDB, ROWB = C::ROWB, REG = C::REG, BUF = C::BUF,
                NI = C::NI, NSTAGE = C::NSTAGE, VSH = C::VSH;
  constexpr int WSTEP = kBf16Waves * 1024;  // bytes one direct load of every wave covers

  // the global-row path needs a K and a V tile of GK keys per wave
  constexpr int LDS_G = (MASK == MASK_LOCAL_GLOBAL) ? kBf16Waves * 2 * GK * ROWB : 0;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * BUF > LDS_G ? NSTAGE * BUF : LDS_G];
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
  const int wph = kBf16Waves / s.HP;              // waves per query head
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
    // every wave of a head holds the head's (up to) 32 global rows; the waves
    // split the keys instead (see the global-row path below)
    const int slot = it.blk * kBf16GlobalRows + l32;
    row_valid = slot < s.n_global;
    q_row = row_valid ? gpos_s[slot] : 0;
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
  auto tile_kt = [&](int iter) { return kt_lo + iter - has_strip; };
  auto is_strip = [&](int iter) { return MASK == MASK_LOCAL_GLOBAL && has_strip && iter == 0; };

  // ---- LDS layout and direct (global -> LDS) tile loads ---------------------
  // A tile region holds BN rows of ROWB bytes, row-major, with the 16-byte
  // chunks of row r permuted: physical chunk = logical chunk ^ swz(r).
  //   K: swz = r & 7         -> the K operand reads (8 consecutive rows, one
  //                              chunk) hit 8 distinct bank groups
  //   V: swz = (r & 3) << VSH -> the transposed reads (4 consecutive rows, two
  //                              chunks) spread over the banks; VSH = 2 where
  //                              a row has 16 chunks (D = 128), else 1
  // A direct load writes 1 KiB: lane l of instruction n of wave w (of W
  // waves) fills slot s = (W*n + w)*64 + l, i.e. row s*16/ROWB and physical
  // chunk (s*16 % ROWB)/16; its source is that row's logical chunk.  Rows
  // advance by W*1024/ROWB per n (a multiple of 8), so the source offset is a
  // per-lane base plus n*W*1024.
  const int slot_b = (wave * 64 + lane) * 16;
  const int srow = slot_b / ROWB, sphys = (slot_b % ROWB) / 16;
  const int k_src = srow * ROWB + (sphys ^ (srow & 7)) * 16;
  const int v_src = srow * ROWB + (sphys ^ ((srow & 3) << VSH)) * 16;

  auto rsrc = [&](const __bf16* base, int kt) {
    // descriptor over rows [kt*BN, S): whole tiles only (tail tiles clamp rows)
    const int row0 = kt * BN;
    const int nbytes = imin(BN, s.S - row0) * ROWB;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)row0 * D), (short)0, nbytes,
                                             0x00020000);
  };
  // rows past S (tail tile) or past n_global (strip) repeat a valid row: their
  // scores are masked, so they carry zero weight
  auto load_region = [&](const __bf16* base, int src_lane, int iter, int dst) {
    if (is_strip(iter)) {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int row = gpos_s[imin(srow + n * (WSTEP / ROWB), s.n_global - 1)];
        const int off = row * ROWB + (src_lane - srow * ROWB);
        dma16_global((const char*)base + off, smem + dst + (n * kBf16Waves + wave) * 1024);
      }
      return;
    }
    const int kt = tile_kt(iter);
    if (kt * BN + BN <= s.S) {
      const __amdgpu_buffer_rsrc_t r = rsrc(base, kt);
#pragma unroll
      for (int n = 0; n < NI; ++n)
        dma16_buffer(r, smem + dst + (n * kBf16Waves + wave) * 1024, src_lane, n * WSTEP);
    } else {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int row = imin(kt * BN + srow + n * (WSTEP / ROWB), s.S - 1);
        const size_t off = (size_t)row * ROWB + (src_lane - srow * ROWB);
        dma16_global((const char*)base + off, smem + dst + (n * kBf16Waves + wave) * 1024);
      }
    }
  };
  auto load_k = [&](int iter, int buf) { load_region(kp, k_src, iter, buf * BUF); };
  auto load_v = [&](int iter, int buf) { load_region(vp, v_src, iter, buf * BUF + REG); };

  // Per-wave tile class.  Tiles EMPTY for this wave (only at the ends of its
  // range, or when it holds no rows) are processed as fully masked.
  auto tile_partial = [&](int iter) -> bool {
    if (!wave_active || is_strip(iter)) return true;
    const int kt = tile_kt(iter);
    if (it.is_global) return kt * BN + BN > s.S;
    return classify_tile(MASK, s.window, s.S, wqa, wqb, kt * BN, BN) != TILE_FULL;
  };

  // ---- operand reads -------------------------------------------------------
  // K operand (key 32*kbk + l32, dims 16*dc + 8*hf + [0,8)): logical chunk
  // 2*dc + hf, physical (2*dc + hf) ^ (l32 & 7) = 2*((dc & 3) ^ (x >> 1)) +
  // (hf ^ (x & 1)) + 8*(dc >> 2) with x = l32 & 7.
  const int kx = l32 & 7;
  int k_rd[4];  // per-lane part for dc & 3; the rest of the offset is an immediate
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4) k_rd[d4] = l32 * ROWB + 16 * (hf ^ (kx & 1)) + 32 * (d4 ^ (kx >> 1));
  auto k_frag = [&](const unsigned char* kbuf, int kbk, int dc) -> bf16x8 {
    return *(const bf16x8*)(kbuf + k_rd[dc & 3] + kbk * 32 * ROWB + 128 * (dc >> 2));
  };
  // V^T operand (dim 32*db + l32, keys 16*pc + 4*hf + [0,4) then +8) from two
  // ds_read_b64_tr_b16 (v_frags): within each 16-lane group, lane 4t + u addresses the
  // 4 dims 32*db + 16*g + 4u of key 16*pc + 4*hf + t (g = lane bit 4), and the
  // transpose hands lane i element (i & 3) of lanes 4t + (i >> 2), t = 0..3,
  // i.e. dim 32*db + l32 of keys 4*hf + t.  Physical chunk of the 4 dims:
  // (4*db + 2*g + (u >> 1)) ^ (t << VSH), which is 4*(db ^ t) + 2*g + (u >> 1)
  // for VSH = 2 and 4*(db ^ (t >> 1)) + 2*(g ^ (t & 1)) + (u >> 1) for VSH = 1
  // (NDB = 2).
  const int tt = (lane >> 2) & 3, uu = lane & 3, gg = (lane >> 4) & 1;
  int v_rd[NDB];  // per-lane part for each db; the 16-key step is an immediate
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    v_rd[db] = (VSH == 2)
                   ? (4 * hf + tt) * ROWB + 64 * (db ^ tt) + 32 * gg + 16 * (uu >> 1) + 8 * (uu & 1)
                   : (4 * hf + tt) * ROWB + 64 * (db ^ (tt >> 1)) + 32 * (gg ^ (tt & 1)) +
                         16 * (uu >> 1) + 8 * (uu & 1);

  // Mask S^T of iteration iter in place.  Register r of block kbk holds key
  // 32*kbk + 8*(r/4) + 4*hf + r%4 of the tile for query q_row.
  auto apply_mask = [&](f32x16* sc, int iter) {
    if (is_strip(iter)) {
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbk * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const int dist = q_row - gpos_s[key];
          const bool vis = key < s.n_global && (dist > s.window || -dist > s.window);
          sc[kbk][r] = vis ? sc[kbk][r] : -INFINITY;
        }
      return;
    }
    // visible keys of this lane's query as an interval of tile-relative
    // indices, shifted by the lane half so each test is against an immediate:
    // lo <= 32*kbk + 8*(r/4) + r%4 <= hi
    long long lo, hi;
    if (it.is_global) { lo = 0; hi = (long long)s.S - 1; }
    else row_interval(MASK, s.window, s.S, q_row, &lo, &hi);
    if (!wave_active) hi = lo - 1;
    const long long base = (long long)tile_kt(iter) * BN + 4 * hf;
    const long long tail = (long long)s.S - 1;
    const long long hi_a = hi < tail ? hi : tail;
    const int lo_r = (int)(lo - base < -1 ? -1 : (lo - base > BN ? BN : lo - base));
    const int hi_r = (int)(hi_a - base < -1 ? -1 : (hi_a - base > BN ? BN : hi_a - base));
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbk * 32 + 8 * (r >> 2) + (r & 3);
        sc[kbk][r] = (key >= lo_r && key <= hi_r) ? sc[kbk][r] : -INFINITY;
      }
  };

  // ---- accumulators --------------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // reference maximum (units of q.k) of query q_row
  float l_run0 = 0.f, l_run1 = 0.f;  // this lane's share of the denominator (two chains)
  const float c = p.c;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  // ---- pipeline ---------------------------------------------------------
  // Tile j lives in stage j % NSTAGE.  Iteration j issues the batch
  // {K(j+3), V(j+2)} (those that exist) into the stages of K(j) and V(j-1),
  // both consumed during iteration j-1.  At the top of iteration j the batch of
  // iteration j-2 (K(j+1), V(j)) must have landed; the batch of iteration j-1
  // may still be in flight, so vmcnt waits down to its size.
  auto wait_batch = [&](int j) {
    // in flight may remain: the batch issued just before iteration j
    if (j + 2 < n_it) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NI));  // vmcnt(2*NI)
    else if (j + 1 < n_it) __builtin_amdgcn_s_waitcnt(0x0f70 | NI);   // vmcnt(NI)
    else __builtin_amdgcn_s_waitcnt(0x0f70);                           // vmcnt(0)
  };
  auto issue_batch = [&](int j) {
    if (j + 3 < n_it) load_k(j + 3, (j + 3) % NSTAGE);
    if (j + 2 < n_it) load_v(j + 2, (j + 2) % NSTAGE);
  };
  if (MASK == MASK_LOCAL_GLOBAL && it.is_global) {
    // ---- global rows: keys split over the waves of a head -----------------
    // The wph waves of a query head hold the same 32 global rows and walk
    // disjoint, contiguous chunks of the S keys, each through its own LDS
    // region (one 32-key K tile and one V tile, same layout and swizzles as
    // the shared ring), so no workgroup barrier is needed inside the walk.
    // K(t+1) is loaded while S(t) is in the softmax, V(t+1) while PV(t) runs.
    constexpr int GREG = GK * ROWB;     // one private K or V tile
    constexpr int NIG = GREG / 1024;    // 1 KiB direct loads per private tile
    constexpr int RPI = 1024 / ROWB;    // tile rows per 1 KiB load
    unsigned char* kreg = smem + wave * 2 * GREG;
    unsigned char* vreg = kreg + GREG;
    const int ntile = cdiv(s.S, GK);
    const int t_lo = (int)((long long)ntile * rpart / wph);
    const int t_hi = (int)((long long)ntile * (rpart + 1) / wph);
    const int lrow = lane * 16 / ROWB, lphys = (lane * 16 % ROWB) / 16;
    auto gload = [&](const __bf16* base, int t, unsigned char* dst, bool is_v) {
#pragma unroll
      for (int n = 0; n < NIG; ++n) {
        const int row = n * RPI + lrow;
        const int key = imin(t * GK + row, s.S - 1);  // tail rows repeat a valid row (masked)
        const int sw = is_v ? ((row & 3) << VSH) : (row & 7);
        dma16_global((const char*)base + (size_t)key * ROWB + (lphys ^ sw) * 16, dst + n * 1024);
      }
    };
    if (t_lo < t_hi) {
      gload(kp, t_lo, kreg, false);
      gload(vp, t_lo, vreg, true);
    }
    for (int t = t_lo; t < t_hi; ++t) {
      const bool more = t + 1 < t_hi;
      __builtin_amdgcn_s_waitcnt(0x0f70 | NIG);  // K(t) landed; V(t) may be in flight
      f32x16 sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) sc = mfma32(k_frag(kreg, 0, dc), qf[dc], sc);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // K operand reads done: the region may be refilled
      if (more) gload(kp, t + 1, kreg, false);
      if ((t + 1) * GK > s.S) {
        // tail tile: keys at or beyond S carry no weight
        const int lim = s.S - t * GK - 4 * hf;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = (8 * (r >> 2) + (r & 3) < lim) ? sc[r] : -INFINITY;
      }
      float mx = max3f(sc[0], sc[1], sc[2]);
      mx = max3f(mx, sc[3], sc[4]);
      mx = max3f(mx, sc[5], sc[6]);
      mx = max3f(mx, sc[7], sc[8]);
      mx = max3f(mx, sc[9], sc[10]);
      mx = max3f(mx, sc[11], sc[12]);
      mx = max3f(mx, sc[13], sc[14]);
      mx = max3f(mx, sc[15], sc[15]);
      mx = pair_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx * c > m_run * c + kLazy) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);
        m_run = m_new;
        l_run0 *= alpha;
        l_run1 *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
      bf16x8 pb[2];
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
          bf16x2 pr;
          pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * pc + u], c, -mc));
          pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * pc + u + 1], c, -mc));
          if (u & 2) l_run1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run1, false);
          else l_run0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run0, false);
          pb[pc][u] = pr[0];
          pb[pc][u + 1] = pr[1];
        }
      if (more) __builtin_amdgcn_s_waitcnt(0x0f70 | NIG);  // V(t) landed; K(t+1) in flight
      else __builtin_amdgcn_s_waitcnt(0x0f70);
      {
        const unsigned vb = lds_addr(vreg);
        bf16x8 fx[NDB], fy[NDB];
        unsigned vbd[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) vbd[db] = vb + v_rd[db];
        v_frags<ROWB, NDB, 0>(fx, vbd);
        v_frags<ROWB, NDB, 1>(fy, vbd);
        lds_wait_frags<2 * NDB>(fx);
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(fx[db], pb[0], oacc[db]);
        lds_wait_frags<0>(fy);
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(fy[db], pb[1], oacc[db]);
      }
      if (more) gload(vp, t + 1, vreg, true);
    }

    // ---- merge the partial (m, l, O) of the waves of each head ------------
    // Fixed pairing (chunk c takes chunk c + half, half = wph/2, wph/4, ...),
    // so results are bitwise reproducible.  In the O^T accumulator lane l of
    // every wave owns the same (query, dims), so partials combine lane by lane:
    //   m = max(m1, m2),  X = X1 * 2^((m1 - m) c) + X2 * 2^((m2 - m) c)  for X in {l, O}.
    // A slot holds one wave's partial: O as 16-byte chunks [chunk][lane], then
    // (m, l) per lane.
    constexpr int SLOT = 4 * NDB * 64 * 16 + 64 * 8;
    static_assert(MASK != MASK_LOCAL_GLOBAL || kBf16Waves / 2 * SLOT <= LDS_G,
                  "merge slots of half the waves fit in LDS");
    const int hh = wave / wph;
    for (int half = wph >> 1; half >= 1; half >>= 1) {
      __syncthreads();  // the private regions (first pass) or slots (later passes) are free
      if (rpart >= half && rpart < 2 * half) {
        unsigned char* sl = smem + (hh * (wph >> 1) + rpart - half) * SLOT;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 x = {oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2],
                              oacc[db][4 * g4 + 3]};
            *(float4*)(sl + ((4 * db + g4) * 64 + lane) * 16) = x;
          }
        *(float2*)(sl + 4 * NDB * 64 * 16 + lane * 8) = float2{m_run, l_run0 + l_run1};
      }
      __syncthreads();
      if (rpart < half) {
        const unsigned char* sl = smem + (hh * (wph >> 1) + rpart) * SLOT;
        const float2 ml = *(const float2*)(sl + 4 * NDB * 64 * 16 + lane * 8);
        const float m_new = fmaxf(m_run, ml.x);
        if (m_new != -INFINITY) {
          const float fa = __builtin_amdgcn_exp2f((m_run - m_new) * c);
          const float fb = __builtin_amdgcn_exp2f((ml.x - m_new) * c);
          l_run0 = (l_run0 + l_run1) * fa + ml.y * fb;
          l_run1 = 0.f;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const float4 x = *(const float4*)(sl + ((4 * db + g4) * 64 + lane) * 16);
              oacc[db][4 * g4] = oacc[db][4 * g4] * fa + x.x * fb;
              oacc[db][4 * g4 + 1] = oacc[db][4 * g4 + 1] * fa + x.y * fb;
              oacc[db][4 * g4 + 2] = oacc[db][4 * g4 + 2] * fa + x.z * fb;
              oacc[db][4 * g4 + 3] = oacc[db][4 * g4 + 3] * fa + x.w * fb;
            }
          m_run = m_new;
        }
      }
    }
  } else {
  f32x16 scur[NKB], snxt[NKB];
  load_k(0, 0);
  load_v(0, 0);
  if (n_it > 1) load_k(1, 1);
  issue_batch(-1);  // K(2), V(1)
  wait_batch(0);
  __syncthreads();
#pragma unroll
  for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
    for (int r = 0; r < 16; ++r) scur[kbk][r] = 0.f;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) scur[kbk] = mfma32(k_frag(smem, kbk, dc), qf[dc], scur[kbk]);

  for (int iter = 0; iter < n_it; ++iter) {
    // Every wave has left the previous tile (its LDS reads are done), and
    // K(j+1), V(j) have landed.
    wait_batch(iter);
    __syncthreads();
    const int cur = iter % NSTAGE, nxt = (iter + 1) % NSTAGE;
    issue_batch(iter);
    const unsigned char* kbuf_nxt = smem + nxt * BUF;      // K(j+1)
    const unsigned char* vbuf_cur = smem + cur * BUF + REG;  // V(j)
    // K(j+1) operands: read two 16-dim steps ahead of their MFMAs
    const unsigned kb = lds_addr(kbuf_nxt);
    const unsigned kbd[4] = {kb + k_rd[0], kb + k_rd[1], kb + k_rd[2], kb + k_rd[3]};
    bf16x8 kf[3][2];
    k_frags<ROWB, 0>(kf[0], kbd);
    k_frags<ROWB, 1>(kf[1], kbd);

    if (tile_partial(iter)) {
      asm volatile("");  // keep this a branch: full tiles skip it
      apply_mask(scur, iter);
    }

    // -- block A: first half of S(j+1) = K(j+1) Q^T beside the row max of S(j).
    //    S(j+1) is always computed; after the last tile it is unused.
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
      for (int r = 0; r < 16; ++r) snxt[kbk][r] = 0.f;
    float mx;
    {
      // four independent v_max3 chains over the 32 scores of this lane, then join
      float t[4];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int kbk = c4 >> 1, rb = (c4 & 1) * 8;
        float x = max3f(scur[kbk][rb], scur[kbk][rb + 1], scur[kbk][rb + 2]);
        x = max3f(x, scur[kbk][rb + 3], scur[kbk][rb + 4]);
        x = max3f(x, scur[kbk][rb + 5], scur[kbk][rb + 6]);
        t[c4] = max3f(x, scur[kbk][rb + 7], scur[kbk][rb + 7]);
      }
      mx = max3f(max3f(t[0], t[1], t[2]), t[3], t[3]);
    }
    s_steps<ROWB, NDC, NDB, 0, NDC / 2>(kf, kbd, qf, snxt);
    mx = pair_max(mx);
    const bool need_rescale = __builtin_amdgcn_ballot_w64(mx * c > m_run * c + kLazy) != 0;

    // rare: a row maximum grew by more than 2^kLazy
    if (need_rescale) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);
      m_run = m_new;
      l_run0 *= alpha;
      l_run1 *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;

    // weights of the 8 registers of one P^T operand -> bf16, added to l
    bf16x8 pb[NPC];
    auto make_p = [&](int pc) {
      const int kbk = pc >> 1, rb = (pc & 1) * 8;
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        bf16x2 pr;
        pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(scur[kbk][rb + t], c, -mc));
        pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(scur[kbk][rb + t + 1], c, -mc));
        // the denominator sums exactly the rounded weights used in P.V
        if (t & 2) l_run1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run1, false);
        else l_run0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run0, false);
        pb[pc][t] = pr[0];
        pb[pc][t + 1] = pr[1];
      }
    };

    // -- block B: second half of S(j+1) beside the first half of P(j); O +=
    //    V(j) P(j) beside the second half of P(j).  The V^T operands of each
    //    16-key step are read one step ahead of their MFMAs.
    const unsigned vb = lds_addr(vbuf_cur);
    unsigned vbd[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vbd[db] = vb + v_rd[db];
    bf16x8 fx[NDB], fy[NDB];
    v_frags<ROWB, NDB, 0>(fx, vbd);
    make_p(0);
    make_p(1);
    s_steps<ROWB, NDC, NDB, NDC / 2, NDC>(kf, kbd, qf, snxt);
    v_frags<ROWB, NDB, 1>(fy, vbd);
    lds_wait_frags<2 * NDB>(fx);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(fx[db], pb[0], oacc[db]);
    v_frags<ROWB, NDB, 2>(fx, vbd);
    lds_wait_frags<2 * NDB>(fy);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(fy[db], pb[1], oacc[db]);
    make_p(2);
    make_p(3);
    v_frags<ROWB, NDB, 3>(fy, vbd);
    lds_wait_frags<2 * NDB>(fx);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(fx[db], pb[2], oacc[db]);
    lds_wait_frags<0>(fy);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(fy[db], pb[3], oacc[db]);
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) scur[kbk] = snxt[kbk];
  }
  }  // shared-ring path

  // ---- epilogue: O = O^T / l, round to bf16, store --------------------------
  {
    const float l_run = l_run0 + l_run1;
    const unsigned lu = __float_as_uint(l_run);
    const float l_other = __uint_as_float(__shfl_xor((int)lu, 32));
    const float l_tot = l_run + l_other;
    // global items: the first wave of each head holds the merged result
    bool store = row_valid && (it.is_global ? rpart == 0 : wave_active);
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
  dim3 grid((unsigned)p.s.n_items), block(kBf16Threads);
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
