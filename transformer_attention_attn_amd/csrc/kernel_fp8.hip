// kernel_fp8.hip -- FP8 (E4M3 or E5M2 inputs) fused attention forward on gfx950
// matrix cores.
//
// The FP8 variant of the tiled online-softmax attention ("Transformer 演进与变
// 体", section Flash Attention, the FlashAttention-3 paragraph: FP8 operands for
// the two matrix products, softmax and accumulation in higher precision):
//   * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (inputs in E4M3 or
//     E5M2, the instruction's operand formats set to match; unit scales, fp32
//     accumulation): 64 dims per instruction.
//   * Online softmax in fp32, as in the bf16 kernel (log2 units, lazy
//     reference maximum), except that the weights come first and the row
//     maximum is computed only when one of them rounds to 2^8 or more (and on
//     a row's first tile).
//   * P is rounded to E4M3 (v_cvt_pk_fp8_f32, round to nearest even; P < 2^8
//     stays below the E4M3 maximum) and O^T += V^T P^T runs on the same
//     instruction (V in the input format, P in E4M3 whatever the inputs:
//     the weights lie in [0, 2^8), where E4M3's third mantissa bit serves
//     and E5M2's range is not needed), 64 keys per instruction; O is
//     accumulated in fp32 and written as bf16.
//   * The denominator is summed on the matrix cores too: l += 1 P^T with an
//     all-ones E4M3 operand (two more instructions per tile), i.e. from the
//     rounded weights, so O is the exact weighted mean under them; the
//     vector ALUs, this kernel's bottleneck, do no sum at all.
//
// gfx950 operand layouts used (checked on the hardware): for the 32x32x64
// FP8 product, lane l holds row (A) or column (B) l % 32 and the 32
// consecutive k indices 32 * (l / 32) + [0, 32), one byte each; the fp32
// accumulator is that of every 32x32 product (lane l: column l % 32, rows
// 8 * (r / 4) + 4 * (l / 32) + r % 4 of register r).  ds_read_b64_tr_b8: in
// each 16-lane group, lane 8h + i receives byte i of the 8-byte rows read by
// the group's lanes 2m + h, m = 0..7, in that order.
//
// Key order.  The A operand of S^T takes K row kappa(rho) for accumulator row
// rho = 8q + 4h + t, with kappa(rho) = 16h + 4q + t, so register r of a 32-key
// block holds key 16 * (l / 32) + r: each lane owns 16 consecutive keys.  For
// O^T += V^T P^T over 64 keys (blocks 2s, 2s+1) the B operand is then the lane's
// own 32 weights in register order, and the V^T operand reads, for each of its
// four 8-byte transposed reads t, the eight keys 64s + 32(t/2) + 16(l/32) +
// 8(t%2) + [0, 8) of its dimension.
//
// Workgroup: eight waves of 32 query rows (query heads of a key/value head
// packed as in the bf16 kernel), 128-key tiles, K and V tiles loaded straight
// into LDS (two stages).  The schedule is the bf16 kernel's ping-pong: two
// wave groups (one wave of each per SIMD) alternate, per barrier-separated
// step, between the matrix block of one tile and the softmax of another, so
// the matrix cores and the vector ALUs of a SIMD work side by side.
//
// LDS swizzles (16-byte chunks of the 128-byte rows): K chunk c of row r sits
// at c ^ g(r), g(r) = ((r >> 1) & 3) | (((r >> 4) & 1) << 2), so the 16 rows a
// 16-lane pass of the K operand reads hit 16 distinct bank groups; V chunk c
// at c ^ (2 * ((r >> 1) & 3)), so the 32 eight-byte pieces a pass of the
// transposed reads touches are distinct.
#include "attn_kernels.h"
#include "gfx950_ops.h"

namespace attn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int F8_D = 128;                 // widest head dimension: bytes of an LDS row
constexpr int F8_BN = 128;                // keys per tile
constexpr int F8_ROWB = F8_D;             // bytes per K or V row
constexpr int F8_REG = F8_BN * F8_ROWB;   // one K or V tile (16 KB)
constexpr int F8_NSTAGE = 2;
constexpr int F8_LOADS = F8_REG / 1024 / 4;  // 1 KiB direct loads per loading wave per tile
constexpr unsigned kE4M3One = 0x38383838u;  // four E4M3 ones
#ifndef F8_OPDEPTH
#define F8_OPDEPTH 3  // LDS operands in flight + 1 in the matrix block
#endif
static_assert(F8_LOADS * 4 * 1024 == F8_REG, "tile split into 1 KiB loads of four waves");

__device__ __forceinline__ int kswz(int row) { return ((row >> 1) & 3) | (((row >> 4) & 1) << 2); }
__device__ __forceinline__ int vswz(int row) { return 2 * ((row >> 1) & 3); }

// Operand formats of the f8f6f4 product: 0 = E4M3, 1 = E5M2 (A, then B).
constexpr int kFmtE4M3 = 0, kFmtE5M2 = 1;
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
}

// Two 16-byte LDS reads at a0 + OFF and a1 + OFF (a 32-byte A operand), as
// inline asm waited for explicitly (the compiler would otherwise wait for the
// direct loads in flight before every LDS read).
template <int OFF>
__device__ __forceinline__ i32x8 lds_read32(unsigned a0, unsigned a1) {
  u32x4 lo, hi;
  asm volatile("ds_read_b128 %0, %2 offset:%4\n\tds_read_b128 %1, %3 offset:%4"
               : "=&v"(lo), "=&v"(hi) : "v"(a0), "v"(a1), "i"(OFF));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
// Four transposed 8-byte reads at base + O0..O3 (a 32-byte V^T operand).
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ i32x8 lds_tr8x4(unsigned base) {
  u32x2 r0, r1, r2, r3;
  asm volatile("ds_read_b64_tr_b8 %0, %4 offset:%5\n\tds_read_b64_tr_b8 %1, %4 offset:%6\n\t"
               "ds_read_b64_tr_b8 %2, %4 offset:%7\n\tds_read_b64_tr_b8 %3, %4 offset:%8"
               : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
               : "v"(base), "i"(O0), "i"(O1), "i"(O2), "i"(O3));
  return i32x8{(int)r0[0], (int)r0[1], (int)r1[0], (int)r1[1], (int)r2[0], (int)r2[1], (int)r3[0], (int)r3[1]};
}
template <int N>
__device__ __forceinline__ void lds_wait8(i32x8& f) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f) : "i"(N));
}

// Row offset (bytes) of transposed read t of 64-key step SK.
constexpr int vrow_off(int SK, int t) { return (64 * SK + 32 * (t >> 1) + 8 * (t & 1)) * F8_ROWB; }

// The matrix block of one step as operand pipelines: operands 0..NV-1 are
// V^T (I = 2 * dim block + 64-key step: O^T += V^T P^T), operands NV..N-1 are
// K (I - NV = 2 * 32-key block + 64-dim step: S^T = K Q^T); the kernel runs
// the P.V part and the S part as two of them.  The LDS reads of
// operand I + DEPTH - 1 are issued before the product of operand I, so
// DEPTH - 1 operands are in flight behind each product; the wait for operand
// I lets the reads issued after it stay outstanding (V: four reads, K: two).
struct BlockOps {
  unsigned vbase[4];            // per-lane V^T read base of each dim block
  unsigned a00, a01, a10, a11;  // per-lane K read addresses (dim step, chunk)
};
template <int NV>
constexpr int reads_of(int i) { return i < NV ? 4 : 2; }
template <int NV>
constexpr int reads_after(int i, int last) {
  int n = 0;
  for (int j = i + 1; j <= last; ++j) n += reads_of<NV>(j);
  return n;
}
template <int I, int NV, int NDC>
__device__ __forceinline__ i32x8 block_read(const BlockOps& o) {
  if constexpr (I < NV) {
    constexpr int DB = I >> 1, SK = I & 1;
    return lds_tr8x4<vrow_off(SK, 0), vrow_off(SK, 1), vrow_off(SK, 2), vrow_off(SK, 3)>(o.vbase[DB]);
  } else {
    constexpr int KBK = (I - NV) / NDC, DC = (I - NV) % NDC;
    return DC == 0 ? lds_read32<KBK * 32 * F8_ROWB>(o.a00, o.a01)
                   : lds_read32<KBK * 32 * F8_ROWB>(o.a10, o.a11);
  }
}
template <int I, int NV, int N, int DEPTH, int FMT, int NDC>
__device__ __forceinline__ void block_step(i32x8 (&op)[DEPTH], const BlockOps& o, const i32x8 (&pf)[2],
                                           const i32x8 (&qf)[2], const i32x8& ones, f32x16 (&oacc)[4],
                                           f32x16& lacc, f32x16 (&sc)[4]) {
  constexpr int J = I + DEPTH - 1;
  if constexpr (J < N) op[J % DEPTH] = block_read<J, NV, NDC>(o);
  constexpr int LAST = J < N ? J : N - 1;
  lds_wait8<reads_after<NV>(I, LAST)>(op[I % DEPTH]);
  if constexpr (I < NV) {
    oacc[I >> 1] = mfma_fp8<FMT, kFmtE4M3>(op[I % DEPTH], pf[I & 1], oacc[I >> 1]);
    // the denominator (no LDS operand) in the shadow of the first reads
    if constexpr (I < 2) lacc = mfma_fp8<kFmtE4M3, kFmtE4M3>(ones, pf[I], lacc);
  } else {
    constexpr int K = I - NV;
    sc[K / NDC] = mfma_fp8<FMT, FMT>(op[I % DEPTH], qf[K % NDC], (K % NDC) ? sc[K / NDC] : f32x16{});
  }
  if constexpr (I + 1 < N) block_step<I + 1, NV, N, DEPTH, FMT, NDC>(op, o, pf, qf, ones, oacc, lacc, sc);
}
template <int NV, int N, int DEPTH, int NDC, int I = 0>
__device__ __forceinline__ void block_prime(i32x8 (&op)[DEPTH], const BlockOps& o) {
  if constexpr (I < DEPTH - 1 && I < N) {
    op[I] = block_read<I, NV, NDC>(o);
    block_prime<NV, N, DEPTH, NDC, I + 1>(op, o);
  }
}
// D: the head dimension (128, or 64: half the P.V and S instructions; the
// LDS rows keep 128 bytes, the upper 64 never read)
template <bool PV, bool S, int FMT, int D>
__device__ __forceinline__ void run_block(const BlockOps& o, const i32x8 (&pf)[2], const i32x8 (&qf)[2],
                                          const i32x8& ones, f32x16 (&oacc)[4], f32x16& lacc,
                                          f32x16 (&sc)[4]) {
  constexpr int NDC = D / 64, NV = PV ? 2 * (D / 32) : 0, N = NV + (S ? 4 * NDC : 0);
  constexpr int DEPTH = F8_OPDEPTH;
  i32x8 op[DEPTH];
  block_prime<NV, N, DEPTH, NDC>(op, o);
  block_step<0, NV, N, DEPTH, FMT, NDC>(op, o, pf, qf, ones, oacc, lacc, sc);
}

// LDS for the global token positions, only in kernels of the local+global mask
template <bool LG>
__device__ __forceinline__ int* f8_gpos_storage() {
  if constexpr (LG) {
    __shared__ int gpos[kMaxGlobal];
    return gpos;
  } else {
    return nullptr;
  }
}

// FMT: the input format of q, k and v (kFmtE4M3 or kFmtE5M2); D: 64 or 128
// (in memory; in LDS every row takes 128 bytes).  MASK_LOCAL_GLOBAL: band
// items see the band |i - j| <= window through their key tiles plus one strip
// tile that gathers the global keys (outside the band only); global-row items
// hold the head's (up to) 32 global rows in every wave of the head, the waves
// take the key tiles in turn (tile kt goes to wave kt % waves-per-head), and
// their partial (m, l, O) merge through LDS in a fixed pairing.
template <int MASK, int FMT, int D>
__global__ __launch_bounds__(kBf16Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8(KParams p) {
  constexpr bool LG = MASK == MASK_LOCAL_GLOBAL;
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int NDB = D / 32, NCH = D / 16;  // 32-dim output blocks, 16-byte chunks per row
  // local+global: a merge slot holds one wave's O (16-byte chunks [chunk][lane])
  // and (m, l) per lane; at most four are written at once
  constexpr int SLOT = NDB * 4 * 64 * 16 + 64 * 8;
  constexpr int TILES_B = F8_NSTAGE * 2 * F8_REG;
  // local+global, global-row items: one private 64-key K tile and V tile per wave
  constexpr int GT = 64, GREG = GT * F8_ROWB, GLOADS = GREG / 1024;
  constexpr int LG_B = (4 * SLOT > kBf16Waves * 2 * GREG) ? 4 * SLOT : kBf16Waves * 2 * GREG;
  constexpr int SMEM_B = (LG && LG_B > TILES_B) ? LG_B : TILES_B;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM_B];
  int* const gpos_s = f8_gpos_storage<LG>();
  const Sched& s = p.s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const Item it = decode_item(s, blockIdx.x);
  if constexpr (LG) {
    if (tid < kMaxGlobal) gpos_s[tid] = tid < s.n_global ? p.gpos[tid] : 0;
    __syncthreads();
  }
  const bool gitem = LG && it.is_global;  // a global-row item (workgroup-uniform)

  // ---- rows of this wave ------------------------------------------------
  const int wph = kBf16Waves / s.HP;
  const int a = it.kvh * s.G + it.hg * s.HP + wave / wph;
  const int rpart = wave % wph;
  const int r0 = gitem ? 0 : it.blk * s.BMh;
  const int r1 = gitem ? s.S - 1 : imin(r0 + s.BMh, s.S) - 1;
  const int q0 = r0 + rpart * 32;
  const int gslot = it.blk * kBf16GlobalRows + l32;  // global items: the lane's global row
  const int q_row = gitem ? (gslot < s.n_global ? gpos_s[gslot] : 0) : q0 + l32;
  const bool row_valid = gitem ? gslot < s.n_global : q_row < s.S;
  const int wqa = gitem ? 0 : q0, wqb = gitem ? s.S - 1 : imin(q0 + 31, s.S - 1);
  const bool wave_active = wqa <= wqb;

  const size_t S = (size_t)s.S;
  const unsigned char* qp = (const unsigned char*)p.q + (size_t)(it.b * s.Hq + a) * S * D;
  const unsigned char* kp = (const unsigned char*)p.k + (size_t)(it.b * s.Hkv + it.kvh) * S * D;
  const unsigned char* vp = (const unsigned char*)p.v + (size_t)(it.b * s.Hkv + it.kvh) * S * D;

  // ---- Q^T operand: lane holds query q_row, dims 64*dc + 32*hf + [0, 32) ----
  i32x8 qf[2];
  {
    const unsigned flip = p.qmode == 1 ? 0x80808080u : 0u;
    const bool zero = p.qmode == 2 || !row_valid;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
      if (!zero && dc < D / 64) {
        const unsigned char* src = qp + (size_t)q_row * D + dc * 64 + hf * 32;
        x0 = *(const u32x4*)src;
        x1 = *(const u32x4*)(src + 16);
      }
      x0 ^= flip;
      x1 ^= flip;
      qf[dc] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                     (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
  }

  // ---- key tiles --------------------------------------------------------
  // (local+global band items: iteration 0 is the strip of global keys)
  int klo, khi;
  key_range(s, gitem ? 1 : 0, r0, r1, &klo, &khi);
  const int kt_lo = klo / F8_BN, kt_hi = khi / F8_BN;
  const int has_strip = (LG && !gitem && s.n_global > 0) ? 1 : 0;
  const int n_it = kt_hi - kt_lo + 1 + has_strip;
  auto tile_kt = [&](int iter) -> int { return kt_lo + iter - has_strip; };
  auto is_strip = [&](int iter) -> bool { return LG && has_strip && iter == 0; };

  // Direct loads, issued by the four waves of group 0: load n of wave gw fills
  // 1 KiB slot sl = gw * F8_LOADS + n of the tile, lane l the 16-byte chunk at
  // row 8 * sl + l / 8, physical chunk l % 8 (its source: that row's logical
  // chunk; at D = 64 logical chunks 4-7 are never read, and their lanes load
  // chunk (logical % 4) of the row, valid memory).  Rows past S repeat the last
  // row (their scores are masked), so tiles past the end of the range load
  // valid memory into a stage that is not read again.
  const int gw = wave & 3;
  const int drow = lane >> 3, dphys = lane & 7;
  // (the strip: row t of the tile is global position t, later rows repeat the
  // last one and are masked)
  auto tile_row = [&](int iter, int trow) -> int {
    if (is_strip(iter)) return gpos_s[imin(trow, s.n_global - 1)];
    return imin(tile_kt(iter) * F8_BN + trow, s.S - 1);
  };
  auto dma_k = [&](int iter, int st) {
#pragma unroll
    for (int n = 0; n < F8_LOADS; ++n) {
      const int trow = 8 * (gw * F8_LOADS + n) + drow;
      const int row = tile_row(iter, trow);
      dma16_global(kp + (size_t)row * D + 16 * ((dphys ^ kswz(trow)) & (NCH - 1)),
                   smem + st * 2 * F8_REG + (gw * F8_LOADS + n) * 1024);
    }
  };
  auto dma_v = [&](int iter, int st) {
#pragma unroll
    for (int n = 0; n < F8_LOADS; ++n) {
      const int trow = 8 * (gw * F8_LOADS + n) + drow;
      const int row = tile_row(iter, trow);
      dma16_global(vp + (size_t)row * D + 16 * ((dphys ^ vswz(trow)) & (NCH - 1)),
                   smem + st * 2 * F8_REG + F8_REG + (gw * F8_LOADS + n) * 1024);
    }
  };

  auto tile_class = [&](int iter) -> int {
    if (!wave_active) return TILE_EMPTY;
    if constexpr (LG) {
      if (gitem) {  // every key, the wave's share of the tiles
        const int kt = tile_kt(iter);
        if (kt % wph != rpart) return TILE_EMPTY;
        return kt * F8_BN + F8_BN > s.S ? TILE_PARTIAL : TILE_FULL;
      }
      if (is_strip(iter)) return TILE_PARTIAL;
    }
    return classify_tile(MASK, s.window, s.S, wqa, wqb, tile_kt(iter) * F8_BN, F8_BN);
  };

  // ---- per-lane LDS read offsets ------------------------------------------
  // K operand (key block kbk, dim step dc): row 32*kbk + kappa(l32), logical
  // chunks 4*dc + 2*hf and + 1 (the block adds an immediate 32*kbk rows: the
  // swizzle depends on row bits 1, 2 and 4 only).
  const int krow = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
  int k_off[2][2];
#pragma unroll
  for (int dc = 0; dc < 2; ++dc)
#pragma unroll
    for (int c = 0; c < 2; ++c) k_off[dc][c] = krow * F8_ROWB + 16 * ((4 * dc + 2 * hf + c) ^ kswz(krow));
  // V^T operand (dim block db, key step sk, read t): this lane addresses row
  // 64*sk + 32*(t/2) + 16*(g/2) + 8*(t%2) + m, 8-byte piece 2*(g%2) + h +
  // 4*db, with g = lane / 16, m = (lane % 16) / 2, h = lane % 2.  The row's
  // bits 1-2 are m's, so the swizzle (pieces ^ 4*((row >> 1) & 3)) is per lane
  // and the (sk, t) part is an immediate row offset.
  const int lg16 = lane >> 4, vm = (lane & 15) >> 1, vh = lane & 1;
  int v_off[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    v_off[db] = F8_REG + (16 * (lg16 >> 1) + vm) * F8_ROWB +
                8 * (2 * (lg16 & 1) + vh + 4 * (db ^ ((vm >> 1) & 3)));

  // ---- accumulators ------------------------------------------------------
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;
  // denominator l = P 1: every register of the accumulator holds the row sum
  // of the lane's query (column l32)
  f32x16 lacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
  const i32x8 ones8 = {(int)kE4M3One, (int)kE4M3One, (int)kE4M3One, (int)kE4M3One,
                       (int)kE4M3One, (int)kE4M3One, (int)kE4M3One, (int)kE4M3One};
  const float c = p.c;

  // ---- the matrix block of one step: O^T += V(jv)^T P^T, then S(js) = K(js) Q^T
  f32x16 sc[4];
  i32x8 pf[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) pf[i] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  auto mfma_block = [&](int jv, bool do_pv, int js, bool do_s) {
    __builtin_amdgcn_s_setprio(1);
    BlockOps o;
    const unsigned vb = lds_addr(smem + (jv & 1) * 2 * F8_REG);
#pragma unroll
    for (int db = 0; db < 4; ++db) o.vbase[db] = vb + v_off[db];
    const unsigned kb = lds_addr(smem + (js & 1) * 2 * F8_REG);
    o.a00 = kb + k_off[0][0];
    o.a01 = kb + k_off[0][1];
    o.a10 = kb + k_off[1][0];
    o.a11 = kb + k_off[1][1];
    // two regions (one pipeline over both would hold too many registers live)
    if (do_pv) run_block<true, false, FMT, D>(o, pf, qf, ones8, oacc, lacc, sc);
    if (do_s) run_block<false, true, FMT, D>(o, pf, qf, ones8, oacc, lacc, sc);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- online softmax of S(j) into the weights pf (E4M3) and l ---------------
  auto softmax = [&](int j, int cls) {
    if (LG && is_strip(j)) {
      // slot t of the strip is global key gpos[t]: seen when it exists and
      // lies outside the row's band (inside, the band tiles hold it)
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbk * 32 + 16 * hf + r;
          const int dist = q_row - gpos_s[imin(key, kMaxGlobal - 1)];
          const bool vis = row_valid && key < s.n_global && (dist > s.window || -dist > s.window);
          sc[kbk][r] = vis ? sc[kbk][r] : -INFINITY;
        }
    } else if (cls == TILE_PARTIAL) {
      // register r of block kbk holds key 32*kbk + 16*hf + r of the tile
      long long lo, hi;
      if (gitem) {
        lo = 0;  // a global row sees every key
        hi = (long long)s.S - 1;
      } else {
        row_interval(MASK, s.window, s.S, q_row, &lo, &hi);
      }
      if (!row_valid) hi = lo - 1;
      const long long base = (long long)tile_kt(j) * F8_BN + 16 * hf;
      const long long hi_a = hi < (long long)s.S - 1 ? hi : (long long)s.S - 1;
      const int lo_r = (int)(lo - base < -1 ? -1 : (lo - base > F8_BN ? F8_BN : lo - base));
      const int hi_r = (int)(hi_a - base < -1 ? -1 : (hi_a - base > F8_BN ? F8_BN : hi_a - base));
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbk * 32 + r;
          sc[kbk][r] = (key >= lo_r && key <= hi_r) ? sc[kbk][r] : -INFINITY;
        }
    }
    // Weights first, against the current reference maximum, when every row of
    // the wave has one; the row maximum (and the rescale) is only needed on a
    // row's first tile and when a weight rounds to 2^8 or more (an E4M3 code
    // with exponent field 15, or the NaN code), and the weights are then
    // recomputed.  Weights stay below 2^8, inside the E4M3 range.
    bool with_max = __builtin_amdgcn_ballot_w64(row_valid && m_run == -INFINITY) != 0;
#pragma nounroll
    for (;;) {
      if (with_max) {
        float mx;
        {
          float t[8];
#pragma unroll
          for (int c4 = 0; c4 < 8; ++c4) {
            const int kbk = c4 >> 1, rb = (c4 & 1) * 8;
            float x = max3f(sc[kbk][rb], sc[kbk][rb + 1], sc[kbk][rb + 2]);
            x = max3f(x, sc[kbk][rb + 3], sc[kbk][rb + 4]);
            x = max3f(x, sc[kbk][rb + 5], sc[kbk][rb + 6]);
            t[c4] = max3f(x, sc[kbk][rb + 7], sc[kbk][rb + 7]);
          }
          mx = max3f(max3f(t[0], t[1], t[2]), max3f(t[3], t[4], t[5]), fmaxf(t[6], t[7]));
        }
        mx = pair_max(mx);
        // a row maximum grew: move the reference to it
        if (__builtin_amdgcn_ballot_w64(mx * c > m_run * c) != 0) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);
          m_run = m_new;
#pragma unroll
          for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
      // bit 7 of a byte of (code + 8) is set exactly for codes 0x78..0x7F
      // (weights are positive: codes below 0x80, no carry between bytes)
      unsigned big = 0u;
      // weights of 64-key step sk: bytes 16*(kbk - 2*sk) + r, four per dword
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r], c, -mc));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r + 1], c, -mc));
          const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r + 2], c, -mc));
          const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r + 3], c, -mc));
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
          big |= (unsigned)w + 0x08080808u;
          pf[kbk >> 1][4 * (kbk & 1) + r / 4] = w;
        }
      if (with_max || __builtin_amdgcn_ballot_w64(row_valid && (big & 0x80808080u) != 0u) == 0)
        break;
      with_max = true;
    }
  };
  auto zero_p = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) pf[i] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  };

  // ---- pipeline (the bf16 kernel's two-stage ping-pong) ----------------------
  // Waves 0-3 (group 0) and 4-7 (group 1), one of each per SIMD.  Per tile two
  // barrier-separated steps; in each, one group runs its matrix block and the
  // other its softmax:
  //   step 2j  : group 0 softmax(S(j))          | group 1 P.V(j-1), S(j)
  //   step 2j+1: group 0 P.V(j), S(j+1); loads  | group 1 softmax(S(j))
  // Tile j lives in stage j % 2.  Group 0 loads K(j+2) and V(j+1) in step
  // 2j+1 (K(j) was last read in step 2j by group 1, V(j-1) in step 2j by group
  // 1) and waits for them at the end of step 2j+2, before the barrier into step
  // 2j+3, the first that reads them.  Group 1 loads nothing.
  // ---- local+global, global-row items: private key walks ------------------
  // Each wave walks its own contiguous run of 64-key tiles through a private
  // LDS region (one K tile and one V tile, the ring's row layout and
  // swizzles), so the waves of a head work on different keys at once and the
  // walk needs no workgroup barrier.  K(t+1) loads during the softmax of tile
  // t, V(t+1) after its P.V; the exact weights use the row maximum of every
  // tile (weights at most 1).
  if (gitem) {
    {
      unsigned char* kreg = smem + wave * 2 * GREG;
      unsigned char* vreg = kreg + GREG;
      const int nt = cdiv(s.S, GT);
      const int t_lo = (int)((long long)nt * rpart / wph);
      const int t_hi = (int)((long long)nt * (rpart + 1) / wph);
      auto gload = [&](int t, bool is_v) {
#pragma unroll
        for (int n = 0; n < GLOADS; ++n) {
          const int trow = 8 * n + drow;
          const int row = imin(t * GT + trow, s.S - 1);
          const int ch = (dphys ^ (is_v ? vswz(trow) : kswz(trow))) & (NCH - 1);
          dma16_global((is_v ? vp : kp) + (size_t)row * D + 16 * ch, (is_v ? vreg : kreg) + n * 1024);
        }
      };
      const unsigned kb = lds_addr(kreg);
      const unsigned ka0 = kb + k_off[0][0], ka1 = kb + k_off[0][1];
      const unsigned kc0 = kb + k_off[1][0], kc1 = kb + k_off[1][1];
      // (v_off counts from the ring's V tile, F8_REG into a stage)
      const unsigned vb = lds_addr(vreg) - (unsigned)F8_REG;
      if (t_lo < t_hi) {
        gload(t_lo, false);
        gload(t_lo, true);
      }
      for (int t = t_lo; t < t_hi; ++t) {
        const bool more = t + 1 < t_hi;
        __builtin_amdgcn_s_waitcnt(0x0f70 | GLOADS);  // K(t) landed; V(t) may be in flight
        {
          const f32x16 zero = {};
          i32x8 k00 = lds_read32<0>(ka0, ka1);
          i32x8 k10 = lds_read32<32 * F8_ROWB>(ka0, ka1);
          lds_wait8<0>(k00);
          lds_wait8<0>(k10);
          sc[0] = mfma_fp8<FMT, FMT>(k00, qf[0], zero);
          sc[1] = mfma_fp8<FMT, FMT>(k10, qf[0], zero);
          if constexpr (D == 128) {
            i32x8 k01 = lds_read32<0>(kc0, kc1);
            i32x8 k11 = lds_read32<32 * F8_ROWB>(kc0, kc1);
            lds_wait8<0>(k01);
            lds_wait8<0>(k11);
            sc[0] = mfma_fp8<FMT, FMT>(k01, qf[1], sc[0]);
            sc[1] = mfma_fp8<FMT, FMT>(k11, qf[1], sc[1]);
          }
        }
        if (more) gload(t + 1, false);  // the K operand reads are done
        // register r of block kbk holds key 32*kbk + 16*hf + r of the tile;
        // keys at or beyond S, and rows past the global count, carry no weight
        const int lim = row_valid ? s.S - t * GT - 16 * hf : 0;
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kbk][r] = (kbk * 32 + r < lim) ? sc[kbk][r] : -INFINITY;
        float mx;
        {
          float t4[4];
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const int kbk = c4 >> 1, rb = (c4 & 1) * 8;
            float x = max3f(sc[kbk][rb], sc[kbk][rb + 1], sc[kbk][rb + 2]);
            x = max3f(x, sc[kbk][rb + 3], sc[kbk][rb + 4]);
            x = max3f(x, sc[kbk][rb + 5], sc[kbk][rb + 6]);
            t4[c4] = fmaxf(x, sc[kbk][rb + 7]);
          }
          mx = max3f(max3f(t4[0], t4[1], t4[2]), t4[3], t4[3]);
        }
        mx = pair_max(mx);
        if (__builtin_amdgcn_ballot_w64(mx * c > m_run * c) != 0) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);
          m_run = m_new;
#pragma unroll
          for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
        i32x8 pw;
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r], c, -mc));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r + 1], c, -mc));
            const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r + 2], c, -mc));
            const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][r + 3], c, -mc));
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
            pw[4 * kbk + r / 4] = w;
          }
        if (more) __builtin_amdgcn_s_waitcnt(0x0f70 | GLOADS);  // V(t) landed; K(t+1) in flight
        else __builtin_amdgcn_s_waitcnt(0x0f70);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          i32x8 vop = lds_tr8x4<vrow_off(0, 0), vrow_off(0, 1), vrow_off(0, 2), vrow_off(0, 3)>(
              vb + (unsigned)v_off[db]);
          lds_wait8<0>(vop);
          oacc[db] = mfma_fp8<FMT, kFmtE4M3>(vop, pw, oacc[db]);
        }
        lacc = mfma_fp8<kFmtE4M3, kFmtE4M3>(ones8, pw, lacc);
        if (more) gload(t + 1, true);  // the V operand reads are done
      }
    }
  } else {
  const int grp = wave >> 2;
  if (grp == 0) {
    dma_k(0, 0);
    dma_v(0, 0);
    dma_k(1, 1);
    __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * F8_LOADS));  // K(0) landed
  }
  __builtin_amdgcn_s_barrier();
  if (grp == 0) {
    if (tile_class(0) != TILE_EMPTY) mfma_block(0, false, 0, true);  // S(0)
    for (int j = 0; j <= n_it; ++j) {
      const int cls = j < n_it ? tile_class(j) : TILE_EMPTY;
      if (cls != TILE_EMPTY) softmax(j, cls);  // step 2j
      else zero_p();
      __builtin_amdgcn_s_waitcnt(0x0f70);  // K(j+1), V(j) landed
      __builtin_amdgcn_s_barrier();
      dma_k(j + 2, j & 1);  // step 2j+1
      dma_v(j + 1, (j + 1) & 1);
      mfma_block(j, cls != TILE_EMPTY, j + 1, j + 1 < n_it && tile_class(j + 1) != TILE_EMPTY);
      __builtin_amdgcn_s_barrier();
    }
  } else {
    for (int j = 0; j <= n_it; ++j) {
      const int cls = j < n_it ? tile_class(j) : TILE_EMPTY;
      mfma_block(j - 1, j >= 1 && tile_class(j - 1) != TILE_EMPTY, j, cls != TILE_EMPTY);  // step 2j
      __builtin_amdgcn_s_barrier();
      if (cls != TILE_EMPTY) softmax(j, cls);  // step 2j+1
      else zero_p();
      __builtin_amdgcn_s_barrier();
    }
  }
  }  // ring pipeline
  __builtin_amdgcn_s_waitcnt(0x0f70);  // no direct load may land after the workgroup ends

  // ---- local+global, global-row items: merge the waves' partial (m, l, O) ----
  // Fixed pairing (wave part r takes part r + half, half = wph/2, wph/4, ...),
  // so results are bitwise reproducible; every wave of a head holds the same
  // rows in the same lanes, so partials combine lane by lane:
  //   m = max(m1, m2),  X = X1 * 2^((m1 - m) c) + X2 * 2^((m2 - m) c)  for X in {l, O}.
  // The first barrier also orders the slots after every wave's last tile read
  // and after every direct load has landed (each wave waited for its own).
  bool store_rows = row_valid && wave_active;
  if constexpr (LG) {
    if (gitem) {
      const int hh = wave / wph;
      for (int half = wph >> 1; half >= 1; half >>= 1) {
        __syncthreads();
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
          *(float2*)(sl + NDB * 4 * 64 * 16 + lane * 8) = float2{m_run, lacc[0]};
        }
        __syncthreads();
        if (rpart < half) {
          const unsigned char* sl = smem + (hh * (wph >> 1) + rpart) * SLOT;
          const float2 ml = *(const float2*)(sl + NDB * 4 * 64 * 16 + lane * 8);
          const float m_new = fmaxf(m_run, ml.x);
          if (m_new != -INFINITY) {
            const float fa = __builtin_amdgcn_exp2f((m_run - m_new) * c);
            const float fb = __builtin_amdgcn_exp2f((ml.x - m_new) * c);
            const float l_new = lacc[0] * fa + ml.y * fb;
#pragma unroll
            for (int r = 0; r < 16; ++r) lacc[r] = l_new;
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
      store_rows = row_valid && rpart == 0;  // the head's first wave holds the merged rows
    } else {
      // band items leave the rows of global queries to the global items
      for (int g = 0; g < s.n_global; ++g) store_rows = store_rows && (gpos_s[g] != q_row);
    }
  }

  // ---- epilogue: O = O^T / l, round to bf16, store --------------------------
  {
    const float l_tot = lacc[0];
    if (store_rows) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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

}  // namespace

template <int FMT, int D>
hipError_t launch_fmt(const KParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.s.n_items), block(kBf16Threads);
  switch (p.s.mask) {
    case MASK_FULL: hipLaunchKernelGGL((attn_fwd_fp8<MASK_FULL, FMT, D>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_fp8<MASK_CAUSAL, FMT, D>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL_WINDOW: hipLaunchKernelGGL((attn_fwd_fp8<MASK_CAUSAL_WINDOW, FMT, D>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((attn_fwd_fp8<MASK_LOCAL_GLOBAL, FMT, D>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_fp8(const KParams& p, int D, bool e5m2, hipStream_t stream) {
  if (D == 64) return e5m2 ? launch_fmt<kFmtE5M2, 64>(p, stream) : launch_fmt<kFmtE4M3, 64>(p, stream);
  return e5m2 ? launch_fmt<kFmtE5M2, 128>(p, stream) : launch_fmt<kFmtE4M3, 128>(p, stream);
}

}  // namespace attn
