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
//   * D = 64 runs two workgroups per CU (the kernel fits in 128 registers
//     and 64 KB of LDS), D = 128 one.
//   * Two wave groups per workgroup (waves 0-3 and 4-7, one of each per
//     SIMD) in ping-pong: per key tile there are two barrier-separated steps,
//     and in each one group runs its matrix block (O += V P for one tile and
//     S = K Q^T for the next) while the other runs its softmax, so the matrix
//     cores and the vector ALUs of a SIMD work side by side.  The wave
//     running its matrix block gets the higher issue priority.
//   * Tile width per head dimension: 64 keys at D = 64 (a block is 32
//     MFMAs), 128 keys at D = 128 (64 MFMAs), which halves the number of
//     barrier-separated steps per key at D = 128.  The source is compiled
//     once per head dimension (ATTN_HEAD_DIM), so each build holds only the
//     constants of its own tile shape.
//   * K and V go straight from HBM into LDS (buffer/global loads with the LDS
//     flag: no staging registers).  D = 64: four-stage rings, group 0 loads
//     the K tiles and group 1 the V tiles.  D = 128: 32 KB tiles, two-stage
//     rings (128 KB), group 0 loads both.  Loads are spread between MFMAs.
//   * LDS operands are read with inline-asm ds_read_b128 (K) and
//     ds_read_b64_tr_b16 (V^T) up to eight MFMAs ahead, with exact lgkmcnt
//     waits: the compiler would otherwise wait for every direct load in
//     flight before each transposed read.  Steps are separated by a bare
//     s_barrier for the same reason (__syncthreads adds a release fence that
//     waits for direct loads); direct loads are covered by explicit vmcnt
//     waits.
//   * The output rescale runs only when a row maximum grows by more than a
//     factor 2^8 (weights stay <= 2^8, far inside bf16/fp32 range); O / l is
//     unchanged by the choice of reference maximum.
//   * Query heads that share a key/value head are packed into one workgroup
//     (up to eight), so each K/V tile is staged once per group.
//   * Fully masked tiles are never visited (mask-aware key-tile ranges); only
//     partial tiles evaluate the per-element mask.
#include "attn_kernels.h"
#include "gfx950_ops.h"

namespace attn {
namespace {

#ifndef ATTN_HEAD_DIM
#error "compile this source once per head dimension: -DATTN_HEAD_DIM=64 or 128"
#endif
// Keys per tile of this build's head dimension.
constexpr int HD = ATTN_HEAD_DIM;
static_assert(HD == 64 || HD == 128, "head dimension 64 or 128");
constexpr int BN = HD == 128 ? 128 : 64;
constexpr int GK = 32;           // keys per private tile of the global-row path
constexpr int NKB = BN / 32;     // 32-key blocks of S^T
constexpr int NPC = BN / 16;     // 16-key reduction steps of O^T
constexpr float kLazy = 8.f;     // rescale threshold, log2 units

// Operand OP of the P.V part of a matrix block: V^T of dims 32*(OP % NDB) +
// l32 for 16-key step OP / NDB (two transposed reads).
template <int ROWB, int NDB, int OP>
__device__ __forceinline__ bf16x8 v_op(const unsigned* vbd) {
  return lds_tr_pair<16 * (OP / NDB) * ROWB, 8 * ROWB>(vbd[OP % NDB]);
}
// Operand OP of the S part: K rows 32*(OP % NKB) + l32 for 16-dim step
// OP / NKB (one read from the per-lane base of that step).
template <int ROWB, int NKB, int OP>
__device__ __forceinline__ bf16x8 k_op(const unsigned* kbd) {
  constexpr int KBK = OP % NKB, DC = OP / NKB;
  return lds_read16<KBK * 32 * ROWB>(kbd[DC]);
}

// s_waitcnt immediate for vmcnt(n) (6-bit count split over two fields) with
// the other counters left unconstrained.
constexpr int vmcnt_enc(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

// Direct loads issued right after MFMA i of a part of l MFMAs that carries
// ndma loads (spread evenly).
constexpr int dma_after(int i, int l, int ndma) {
  int c = 0;
  for (int k = 0; k < ndma; ++k)
    if (((k + 1) * l) / (ndma + 1) - 1 == i) ++c;
  return c;
}
template <int M>
struct ModeC {
  static constexpr int value = M;
};
// The operand sequence of a matrix block.  MODE 0: P.V only (O^T += V^T P^T
// over the NDB output blocks, 2*NKB 16-key steps); MODE 1: S only (S^T = K Q^T
// over the NKB 32-key blocks); MODE 2: P.V then S as one sequence, so the K
// operands of S are read while the last P.V MFMAs run.
template <int MODE, int NDB, int NDC, int NKB>
struct BlockSeq {
  static constexpr int NPV = 2 * NKB * NDB, NSM = NKB * NDC;
  static constexpr int L = MODE == 0 ? NPV : MODE == 1 ? NSM : NPV + NSM;
  static constexpr bool is_pv(int i) { return MODE == 0 || (MODE == 2 && i < NPV); }
  static constexpr int s_index(int i) { return MODE == 1 ? i : i - NPV; }
  static constexpr int reads(int i) { return is_pv(i) ? 2 : 1; }
  // LDS reads issued after operand i when MFMA i waits for it: the operands
  // i+1 .. i+pf-1 of the ring
  static constexpr int younger(int i, int pf) {
    int n = 0;
    for (int k = i + 1; k < i + pf && k < L; ++k) n += reads(k);
    return n;
  }
};

template <int MODE, int ROWB, int NDB, int NDC, int NKB, int OP>
__device__ __forceinline__ bf16x8 block_op(const unsigned* vbd, const unsigned* kbd) {
  using Q = BlockSeq<MODE, NDB, NDC, NKB>;
  if constexpr (Q::is_pv(OP)) return v_op<ROWB, NDB, OP>(vbd);
  else return k_op<ROWB, NKB, Q::s_index(OP)>(kbd);
}

// MFMAs [I, L) of a matrix block: wait for operand I, MFMA I, read operand
// I + PF into the freed ring slot, then the direct loads scheduled after MFMA I.
template <int MODE, int ROWB, int NDB, int NDC, int NKB, int PF, int I, int NDMA, typename Dma>
__device__ __forceinline__ void block_steps(bf16x8 (&ring)[PF], const unsigned* vbd,
                                            const unsigned* kbd, const bf16x8* pb,
                                            const bf16x8* qf, f32x16* oacc, f32x16* sc,
                                            Dma& dma) {
  using Q = BlockSeq<MODE, NDB, NDC, NKB>;
  if constexpr (I < Q::L) {
    static_assert(Q::younger(I, PF) <= 15, "lgkmcnt holds at most 15");
    lds_wait1<Q::younger(I, PF)>(ring[I % PF]);
    if constexpr (Q::is_pv(I)) {
      oacc[I % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[I % PF], pb[I / NDB],
                                                              oacc[I % NDB], 0, 0, 0);
    } else {
      constexpr int J = Q::s_index(I);
      if constexpr (J / NKB == 0)
        sc[J % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[I % PF], qf[0], f32x16{}, 0, 0, 0);
      else
        sc[J % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[I % PF], qf[J / NKB],
                                                              sc[J % NKB], 0, 0, 0);
    }
    if constexpr (I + PF < Q::L) ring[I % PF] = block_op<MODE, ROWB, NDB, NDC, NKB, I + PF>(vbd, kbd);
    dma(dma_after(I, Q::L, NDMA));
    block_steps<MODE, ROWB, NDB, NDC, NKB, PF, I + 1, NDMA>(ring, vbd, kbd, pb, qf, oacc, sc, dma);
  }
}
template <int MODE, int ROWB, int NDB, int NDC, int NKB, int PF, int I>
__device__ __forceinline__ void block_prime(bf16x8 (&ring)[PF], const unsigned* vbd,
                                            const unsigned* kbd) {
  if constexpr (I < PF) {
    ring[I] = block_op<MODE, ROWB, NDB, NDC, NKB, I>(vbd, kbd);
    block_prime<MODE, ROWB, NDB, NDC, NKB, PF, I + 1>(ring, vbd, kbd);
  }
}
template <int MODE, int ROWB, int NDB, int NDC, int NKB, int NDMA, typename Dma>
__device__ __forceinline__ void block_run(const unsigned* vbd, const unsigned* kbd,
                                          const bf16x8* pb, const bf16x8* qf, f32x16* oacc,
                                          f32x16* sc, Dma& dma) {
  constexpr int L = BlockSeq<MODE, NDB, NDC, NKB>::L;
  // operands in flight (at most 7 * 2 reads outstanding); four at D = 64 to
  // stay within 128 registers
  constexpr int PFMAX = HD == 64 ? 4 : 8;
  constexpr int PF = L < PFMAX ? L : PFMAX;
  bf16x8 ring[PF];
  block_prime<MODE, ROWB, NDB, NDC, NKB, PF, 0>(ring, vbd, kbd);
  block_steps<MODE, ROWB, NDB, NDC, NKB, PF, 0, NDMA>(ring, vbd, kbd, pb, qf, oacc, sc, dma);
}

// The lane id, read afresh: values derived from it are recomputed where used
// instead of being held (and spilled) across the persistent kernel's items.
__device__ __forceinline__ unsigned fresh_lane() {
  unsigned l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// A buffer descriptor over [base, base + bytes) built from wave-uniform
// values: the fields are read from the first lane, so the descriptor sits in
// scalar registers even where the compiler cannot prove them uniform (a
// descriptor in vector registers turns every access into a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const unsigned long long a = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((unsigned long long)hi << 32) | lo), (short)0,
                                           n, 0x00020000);
}

// Persistent launches (one workgroup per CU): round k of workgroup w takes
// item k*W + w on even rounds and the mirrored slot on odd rounds, mirrored
// in groups of eight so that the item's id modulo 8 (its key/value head when
// there are eight pairs) stays w % 8, the XCD the workgroup runs on.  With the
// causal heaviest-first order the mirrored rounds pair long items with short
// ones, so the workgroups' tile counts come out nearly equal.  -1: no item.
__device__ __forceinline__ int pers_item_id(int k, int w, int W, int n_items) {
  int slot = w;
  if (k & 1) slot = (W % 8 == 0) ? (W - 8 - (w & ~7)) + (w & 7) : W - 1 - w;
  const long long id = (long long)k * W + slot;
  return id < n_items ? (int)id : -1;
}

template <int D>
struct Cfg {
  static constexpr int NDC = D / 16;            // 16-dim reduction steps of S^T
  static constexpr int NDB = D / 32;            // 32-dim blocks of O^T
  static constexpr int ROWB = D * 2;            // bytes per K or V row
  static constexpr int REG = BN * ROWB;         // bytes of one K or V tile
  static constexpr int VSH = D == 128 ? 2 : 1;  // V chunk swizzle shift
  // K chunk swizzle: the 16 rows that one 16-lane pass of a 16-byte operand
  // read touches land on 16 distinct 16-byte bank groups of the 64 LDS banks
  static __host__ __device__ constexpr int ksw(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
  }
  static constexpr int BUF = 2 * REG;           // K tile then V tile
  static constexpr int NSTAGE = BN == 128 ? 2 : 4;  // LDS stages of the K/V ring
  static constexpr int NGL = REG / 1024 / 4;    // 1 KiB direct loads per wave per tile (4 waves)
  static constexpr int RSTEP = 4096 / ROWB;     // rows between a lane's successive loads
  static_assert(NGL * 4 * 1024 == REG && RSTEP % 8 == 0, "tile split into 1 KiB group loads");
  static_assert(NSTAGE * BUF <= 160 * 1024, "LDS budget of one CU");
};

// Waves per SIMD: one workgroup per CU at D = 128 (two waves per SIMD, up to
// 256 registers each); two at D = 64, whose kernel fits in 128 registers and
// 64 KB of LDS, so a second workgroup fills the gaps of the first.
constexpr int kWavesPerEu = HD == 64 ? 4 : 2;
// GEN = 0: attn_fwd's dense square layout.  GEN = 1: the general form behind
// attn_fwd_ex -- Sq query rows (s.S) against Sk keys (s.Sk), query i at key
// position i + s.off, element strides for the batch, head and row dimensions
// of each tensor, optional per-sequence lengths (right padding); under the
// local+global mask the global indices are key positions (a global query is
// row gpos - off of its sequence).  GEN = 2: GEN = 1 plus the ALiBi
// bias.  GEN = 3: GEN = 1 with a block-sparse layout (square, no lengths,
// at most kSparseShortKeys positions); GEN = 5: the same up to kSparseMaxKeys
// (a longer tile list).
// GEN = 4: GEN = 1 plus a distance-bias table (masks FULL, CAUSAL and
// CAUSAL_WINDOW).
// LDS for the global token positions, only in kernels of the local+global
// mask (the persistent kernels use all 160 KB otherwise)
template <bool LG>
__device__ __forceinline__ int* gpos_storage() {
  if constexpr (LG) {
    __shared__ int gpos[kMaxGlobal];
    return gpos;
  } else {
    return nullptr;
  }
}

template <int D, int MASK, int GEN = 0, int PERS = 0>
__global__ __launch_bounds__(kBf16Threads) __attribute__((amdgpu_waves_per_eu(kWavesPerEu, kWavesPerEu)))
void attn_fwd_bf16(KParams p_arg) {
  using C = Cfg<D>;
  constexpr bool ALIBI = GEN == 2;
  constexpr bool SPARSE = GEN == 3 || GEN == 5;
  constexpr bool DBIAS = GEN == 4;
  constexpr int NDC = C::NDC, NDB = C::NDB, ROWB = C::ROWB, REG = C::REG, BUF = C::BUF,
                NGL = C::NGL, RSTEP = C::RSTEP, NSTAGE = C::NSTAGE, VSH = C::VSH;

  // the global-row path needs a K and a V tile of GK keys per wave
  constexpr int LDS_G = (MASK == MASK_LOCAL_GLOBAL) ? kBf16Waves * 2 * GK * ROWB : 0;
  constexpr int LDS_MAIN = NSTAGE * BUF > LDS_G ? NSTAGE * BUF : LDS_G;
  // PERS: the next item's Q of wave group 0 (32 rows per wave, laid out like
  // the first 32 rows of a K tile)
  constexpr int LDS_Q = PERS ? 4 * 32 * ROWB : 0;
  // DBIAS: per wave, the table entries one tile's scores of its 32 rows use
  // (BN + 31 consecutive distances), loaded 64 entries per direct load
  constexpr int NBD = (BN + 31 + 63) / 64;
  constexpr int LDS_B = DBIAS ? kBf16Waves * NBD * 256 : 0;
  static_assert(LDS_MAIN + LDS_Q + LDS_B + (MASK == MASK_LOCAL_GLOBAL ? kMaxGlobal * 4 : 0) <=
                    160 * 1024,
                "LDS budget of one CU");
  static_assert(!DBIAS || (!PERS && MASK != MASK_LOCAL_GLOBAL), "distance bias: general masks");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_MAIN + LDS_Q + LDS_B];
  int* const gpos_s = gpos_storage<MASK == MASK_LOCAL_GLOBAL>();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int grp = wave >> 2;  // wave group of the ping-pong schedule
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // lane half: selects the k sub-range of an MFMA operand
  if (MASK == MASK_LOCAL_GLOBAL) {
    if (tid < kMaxGlobal) gpos_s[tid] = tid < p_arg.s.n_global ? p_arg.gpos[tid] : 0;
    __syncthreads();
  }
  // PERS: the workgroup walks its list of items (see pers_item_id); else it
  // runs the one item blockIdx.x.  The key/value tiles of consecutive items
  // form one stream (gofs: the place of this item's first tile in it; stream
  // tile t lives in stage t % NSTAGE).
  int gofs = 0;
  // PERS: the items of this and the next two rounds, decoded once each and
  // carried from round to round (id < 0: none)
  int id_n1 = -1, id_n2 = -1;
  Item it_n1{}, it_n2{};
  bf16x8 qf[NDC];  // Q^T operand of the current item
  for (int round = 0; PERS || round == 0; ++round) {
  // PERS: the arguments are read again for every item from the kernel
  // argument segment, through a pointer the compiler cannot see through, so
  // nothing derived from them is held in registers across items (the item's
  // code runs at the register limit of two waves per SIMD)
  typedef const __attribute__((address_space(4))) KParams* KArgPtr;
  KArgPtr kap = (KArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
  if constexpr (PERS) asm volatile("" : "+s"(kap));
  KParams p_item;
  __builtin_memcpy(&p_item, (const KParams*)kap, sizeof(KParams));
  const KParams& p = PERS ? p_item : p_arg;
  const Sched& s = p.s;
  Item it;
  if constexpr (PERS) {
    if (round == 0) {
      const int id0 = pers_item_id(0, blockIdx.x, gridDim.x, (int)s.n_items);
      if (id0 < 0) break;
      it = decode_item(s, id0);
      id_n1 = pers_item_id(1, blockIdx.x, gridDim.x, (int)s.n_items);
      if (id_n1 >= 0) it_n1 = decode_item(s, id_n1);
    } else {
      if (id_n1 < 0) break;
      it = it_n1;
      id_n1 = id_n2;
      it_n1 = it_n2;
    }
    id_n2 = id_n1 >= 0 ? pers_item_id(round + 2, blockIdx.x, gridDim.x, (int)s.n_items) : -1;
    if (id_n2 >= 0) it_n2 = decode_item(s, id_n2);
  } else {
    it = decode_item(s, blockIdx.x);
  }
  // valid query rows SQ and keys SK of this sequence, and the key position
  // OFF of query row 0 (GEN: queries aligned to the end of the keys; with
  // per-sequence lengths the rest of the rows and keys are padding)
  int SQ = s.S, SK = GEN ? s.Sk : s.S, OFF = GEN ? s.off : 0;
  if constexpr (GEN != 0) {
    if (p.qlen) SQ = imin(imax(p.qlen[it.b], 0), s.S);
    if (p.kvlen) SK = imin(imax(p.kvlen[it.b], 0), s.Sk);
    OFF = SK - SQ;
  }
  const int SKA = GEN ? imax(SK, 1) : SK;  // rows addressed by the tile loads (row 0 always exists)

  // ---- rows of this wave -------------------------------------------------
  const int wph = kBf16Waves / s.HP;              // waves per query head
  const int a = it.kvh * s.G + it.hg * s.HP + wave / wph;
  const int rpart = wave % wph;
  int q_row, wqa = 0, wqb = -1, r0 = 0, r1 = 0;
  bool row_valid;
  if (!it.is_global) {
    r0 = it.blk * s.BMh;
    r1 = imin(r0 + s.BMh, SQ) - 1;
    const int q0 = r0 + rpart * 32;
    q_row = q0 + (PERS ? (int)(fresh_lane() & 31) : l32);
    row_valid = q_row < SQ;
    wqa = q0;
    wqb = imin(q0 + 31, SQ - 1);
  } else {
    // every wave of a head holds the head's (up to) 32 global rows; the waves
    // split the keys instead (see the global-row path below).  The global
    // indices are key positions: query row gpos - OFF, present when that row
    // and that key exist in this sequence.
    const int slot = it.blk * kBf16GlobalRows + l32;
    const int gp = slot < s.n_global ? gpos_s[slot] : -1;
    row_valid = gp >= 0 && gp < SK && gp - OFF >= 0 && gp - OFF < SQ;
    q_row = row_valid ? gp - OFF : 0;
  }
  const bool wave_active = wqa <= wqb;
  // key positions of the wave's first and last valid rows
  const int wpa = wqa + OFF, wpb = wqb + OFF;
  // GEN: the wave also holds padded query rows (masked on every tile)
  const bool wave_pad = GEN && wave_active && imin(wqa + 31, s.S - 1) >= SQ;
  // ALiBi: the head's slope in units of the scores below (q.k, or log2 units
  // when the scale is zero), and this lane's query position
  float slope_u = 0.f;
  if constexpr (ALIBI) slope_u = p.slopes[a] * p.bias_k;
  const int q_pos = q_row + OFF;

  const size_t S = (size_t)s.S;
  const __bf16* qp;
  const __bf16* kp;
  const __bf16* vp;
  if constexpr (GEN) {
    qp = (const __bf16*)p.q + it.b * p.qs[0] + a * p.qs[1];
    kp = (const __bf16*)p.k + it.b * p.ks[0] + it.kvh * p.ks[1];
    vp = (const __bf16*)p.v + it.b * p.vs[0] + it.kvh * p.vs[1];
  } else {
    qp = (const __bf16*)p.q + (size_t)(it.b * s.Hq + a) * S * D;
    kp = (const __bf16*)p.k + (size_t)(it.b * s.Hkv + it.kvh) * S * D;
    vp = (const __bf16*)p.v + (size_t)(it.b * s.Hkv + it.kvh) * S * D;
  }
  // bytes between consecutive K and V rows
  const int KRB = GEN ? (int)p.ks[2] * 2 : ROWB, VRB = GEN ? (int)p.vs[2] * 2 : ROWB;

  // ---- Q^T operand: lane holds query q_row, dims 16*dc + 8*hf + [0, 8) -----
  // PERS: loaded inside each wave group's part of the schedule (see below)
  auto load_q_global = [&]() {
    // (the persistent kernel runs with plain Q only)
    const u32x4 flip = (!PERS && p.qmode == 1)
                           ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                           : u32x4{0u, 0u, 0u, 0u};
    const bool zero = (!PERS && p.qmode == 2) || !row_valid;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (!zero) x = *(const u32x4*)(qp + (size_t)q_row * (GEN ? p.qs[2] : D) + dc * 16 + hf * 8);
      x ^= flip;
      qf[dc] = __builtin_bit_cast(bf16x8, x);
    }
  };
  if constexpr (!PERS) load_q_global();

  // ---- block-sparse tile list (GEN = 3) ------------------------------------
  // The item's key tiles in order, one per lane of lv[c] (64 per register):
  // the tile index in bits 0-15 and, for each 64-row query block the item
  // spans (slot = block - first block, at most four), which of the tile's
  // 64-key halves that block may see, at bits 16 + 2*slot (both bits for a
  // 64-key tile).  Tiles past the item's last row are left out under the
  // causal mask.  Every wave builds the same list (no LDS, no barrier).
  constexpr int NLV = SPARSE ? ((GEN == 5 ? kSparseMaxKeys : kSparseShortKeys) / BN + 63) / 64 : 1;
  unsigned lv[NLV];
  int n_lv[NLV];
  int n_list = 0;
  const int wslot = (wqa >> 6) - (r0 >> 6);  // this wave's query block slot
  if constexpr (SPARSE) {
    const int qb0 = r0 >> 6, nqs = (r1 >> 6) - qb0 + 1;
    const int nkt = cdiv(SK, BN);
    const int kt_end = MASK == MASK_CAUSAL ? imin(nkt, r1 / BN + 1) : nkt;
#pragma unroll
    for (int c = 0; c < NLV; ++c) {
      const int kt = c * 64 + lane;
      unsigned e = 0;
      if (kt < kt_end) {
        unsigned codes = 0;
        for (int sl = 0; sl < nqs; ++sl) {
          const unsigned* row = p.layout + (size_t)(qb0 + sl) * p.lay_nw;
          const unsigned cd = BN == 128 ? (row[kt >> 4] >> ((2 * kt) & 31)) & 3u
                                        : ((row[kt >> 5] >> (kt & 31)) & 1u) * 3u;
          codes |= cd << (2 * sl);
        }
        if (codes) e = (unsigned)kt | (codes << 16);
      }
      // lanes holding a tile move to the front in order, the others behind
      const unsigned long long m = __builtin_amdgcn_ballot_w64(e != 0u);
      const int below = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
      const int cnt = __builtin_popcountll(m);
      const int dst = e ? below : cnt + (lane - below);
      lv[c] = (unsigned)__builtin_amdgcn_ds_permute(dst * 4, (int)e);
      n_lv[c] = cnt;
      n_list += cnt;
    }
  }
  // list entry of iteration iter (past the end: the last one; tile 0 if none):
  // register c holds entries [sum of n_lv below c, + n_lv[c]) in its first lanes
  auto entry = [&](int iter) -> unsigned {
    int t = imax(imin(iter, n_list - 1), 0);
    if constexpr (NLV <= 2) {
      if (NLV == 1 || t < n_lv[0]) return (unsigned)__builtin_amdgcn_readlane((int)lv[0], t);
      return (unsigned)__builtin_amdgcn_readlane((int)lv[NLV - 1], t - n_lv[0]);
    }
    unsigned e = (unsigned)__builtin_amdgcn_readlane((int)lv[0], imin(t, 63));
#pragma unroll
    for (int c = 1; c < NLV; ++c) {
      t -= n_lv[c - 1];
      if (t >= 0 && t < n_lv[c]) e = (unsigned)__builtin_amdgcn_readlane((int)lv[c], t);
    }
    return e;
  };
  auto wave_code = [&](int iter) -> unsigned { return (entry(iter) >> (16 + 2 * wslot)) & 3u; };

  // ---- key tiles to visit ------------------------------------------------
  int klo = 0, khi = -1;
  if constexpr (SPARSE) {
  } else if constexpr (GEN) {
    // keys seen by the valid rows r0..r1 at key positions r0 + OFF .. r1 + OFF
    // (local+global: the band part; the global keys come in the strip tile)
    const int pa = r0 + OFF, pb = r1 + OFF;
    if (MASK == MASK_LOCAL_GLOBAL) {
      klo = it.is_global ? 0 : imax(0, pa - s.window);
      khi = it.is_global ? SK - 1 : (int)(pb + (long long)s.window < SK ? pb + s.window : SK - 1);
    } else {
      klo = MASK == MASK_CAUSAL_WINDOW ? imax(0, pa - s.window + 1) : 0;
      khi = MASK == MASK_FULL ? SK - 1 : imin(pb, SK - 1);
    }
  } else {
    key_range(s, it.is_global, r0, r1, &klo, &khi);
  }
  const int kt_lo = klo / BN, kt_hi = khi / BN;
  // PERS: the first tiles of the next two items (the loads run two tiles
  // ahead, across item boundaries): key/value head index b * Hkv + kvh (-1:
  // none), first tile, tile count
  int nx_kv = -1, nx_lo = 0, nx_n = 0, nx2_kv = -1, nx2_lo = 0;
  if constexpr (PERS) {
    if (id_n1 >= 0) {
      const int a0 = it_n1.blk * s.BMh, a1 = imin(a0 + s.BMh, s.S) - 1;
      int lo1, hi1;
      key_range(s, 0, a0, a1, &lo1, &hi1);
      nx_kv = it_n1.b * s.Hkv + it_n1.kvh;
      nx_lo = lo1 / BN;
      nx_n = hi1 / BN - nx_lo + 1;
      if (id_n2 >= 0) {
        const int b0 = it_n2.blk * s.BMh, b1 = imin(b0 + s.BMh, s.S) - 1;
        int lo2, hi2;
        key_range(s, 0, b0, b1, &lo2, &hi2);
        nx2_kv = it_n2.b * s.Hkv + it_n2.kvh;
        nx2_lo = lo2 / BN;
      }
    }
  }
  const int has_strip = (MASK == MASK_LOCAL_GLOBAL && !it.is_global && s.n_global > 0) ? 1 : 0;
  // GEN: an item of padded rows, or of a sequence without keys, visits
  // nothing; rows that see no band key (positions before the first key)
  // still visit the strip of global keys
  const int n_it = SPARSE ? n_list
                   : !GEN ? (kt_hi - kt_lo + 1) + has_strip
                   : (r1 < r0 || SK == 0) ? 0
                   : (khi < klo ? 0 : kt_hi - kt_lo + 1) + has_strip;
  auto tile_kt = [&](int iter) -> int {
    if constexpr (SPARSE) return (int)(entry(iter) & 0xffffu);
    return kt_lo + iter - has_strip;
  };
  auto is_strip = [&](int iter) { return MASK == MASK_LOCAL_GLOBAL && has_strip && iter == 0; };

  // ---- LDS layout and direct (global -> LDS) tile loads ---------------------
  // A tile region holds BN rows of ROWB bytes, row-major, with the 16-byte
  // chunks of row r permuted: physical chunk = logical chunk ^ swz(r).
  //   K: swz = ksw(r)        -> the K operand reads (16 consecutive rows, one
  //                              chunk) hit 16 distinct bank groups
  //   V: swz = (r & 3) << VSH -> the transposed reads (4 consecutive rows, two
  //                              chunks) spread over the banks; VSH = 2 where
  //                              a row has 16 chunks (D = 128), else 1
  // K tiles are loaded by wave group 0 (waves 0-3) and V tiles by group 1.
  // A direct load writes 1 KiB: lane l of load n of wave gw (0..3 in its
  // group) fills slot s = (4n + gw)*64 + l, i.e. row s*16/ROWB and physical
  // chunk (s*16 % ROWB)/16; its source is that row's logical chunk.  Rows
  // advance by RSTEP (a multiple of 8) per n, so the source column is fixed
  // per lane.
  const int gw = wave & 3;
  const int slot_b = (gw * 64 + lane) * 16;
  const int srow = slot_b / ROWB, sphys = (slot_b % ROWB) / 16;
  const int k_col = (sphys ^ C::ksw(srow)) * 16;
  const int v_col = (sphys ^ ((srow & 3) << VSH)) * 16;
  // Load n of this wave for tile iter of K (isk) or V into stage st.  Rows past
  // the sequence's keys (tail tile; strip entries past n_global, or GEN: at a
  // padded position) repeat a valid row: their scores are masked, so they
  // carry zero weight, and what padding holds is never multiplied in.  Tiles
  // past the end of the range load clamped rows into a stage that is not read
  // again.
  auto dma = [&](bool isk, int iter, int st, int n) {
    int row;
    if (is_strip(iter)) row = imin(gpos_s[imin(srow + n * RSTEP, s.n_global - 1)], SKA - 1);
    else row = imin(tile_kt(iter) * BN + srow + n * RSTEP, SKA - 1);
    const char* src = (const char*)(isk ? kp : vp) + (size_t)row * (isk ? KRB : VRB) + (isk ? k_col : v_col);
    dma16_global(src, smem + (isk ? 0 : NSTAGE * REG) + st * REG + (n * 4 + gw) * 1024);
  };
  // in-loop form (iter >= 1, never the strip): a buffer descriptor over the
  // tile's valid rows and a 32-bit lane offset clamped to the last valid row,
  // so no lane is out of range.
  const int k_off = srow * KRB + k_col, v_off = srow * VRB + v_col;
  // PERS: byte bases of the next two items' key and value rows
  const char* nx_k = nullptr;
  const char* nx_v = nullptr;
  const char* nx2_k = nullptr;
  const char* nx2_v = nullptr;
  if constexpr (PERS) {
    if (nx_kv >= 0) {
      nx_k = (const char*)p.k + (size_t)nx_kv * S * ROWB;
      nx_v = (const char*)p.v + (size_t)nx_kv * S * ROWB;
    }
    if (nx2_kv >= 0) {
      nx2_k = (const char*)p.k + (size_t)nx2_kv * S * ROWB;
      nx2_v = (const char*)p.v + (size_t)nx2_kv * S * ROWB;
    }
  }
  // The buffer descriptor of one K or V tile (iter: the item's tile index;
  // PERS: tiles past the item's last are the next items' first tiles) over
  // its valid rows, with the offset clamp of its last valid row.  Built once
  // per block, shared by the block's direct loads of that tile.
  struct TileRsrc {
    __amdgpu_buffer_rsrc_t r;
    int lclamp;
  };
  auto tile_rsrc = [&](bool isk, int iter) -> TileRsrc {
    const char* base = (const char*)(isk ? kp : vp);
    int kt = tile_kt(iter);
    TileRsrc t;
    if constexpr (PERS) {
      if (iter >= n_it) {
        if (iter - n_it < nx_n) {
          base = isk ? nx_k : nx_v;
          kt = nx_lo + iter - n_it;
        } else {
          base = isk ? nx2_k : nx2_v;
          kt = nx2_lo;
        }
        if (base == nullptr) {
          // past the end of the stream: a descriptor of no bytes (its loads
          // are out of range and read nothing) into a stage read no more
          t.r = __builtin_amdgcn_make_buffer_rsrc((void*)p.k, (short)0, 0, 0x00020000);
          t.lclamp = 0;
          return t;
        }
      }
    }
    // tiles past the last one of the sequence load the last tile instead
    const int row0 = imin(kt, (SKA - 1) / BN) * BN;
    const int nrows = imin(SKA - row0, BN);
    const int RB = isk ? KRB : VRB;
    t.r = __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)row0 * RB), (short)0,
                                            (nrows - 1) * RB + ROWB, 0x00020000);
    // (the lane's column is opaque here: the sum is formed per tile instead
    // of the compiler keeping a column-minus-row constant live)
    int col = isk ? k_col : v_col;
    asm volatile("" : "+v"(col));
    t.lclamp = (nrows - 1) * RB + col;
    return t;
  };
  auto dma_tile_at = [&](bool isk, const TileRsrc& t, int st, int n, int lb) {
    const int RB = isk ? KRB : VRB;
    const int off = imin(lb + n * RSTEP * RB, t.lclamp);
    dma16_buffer(t.r, smem + (isk ? 0 : NSTAGE * REG) + st * REG + (n * 4 + gw) * 1024, off, 0);
  };
  auto dma_tile = [&](bool isk, const TileRsrc& t, int st, int n) {
    dma_tile_at(isk, t, st, n, isk ? k_off : v_off);
  };
  auto dma_band = [&](bool isk, int iter, int st, int n) { dma_tile(isk, tile_rsrc(isk, iter), st, n); };

  // Per-wave tile class.  Tiles EMPTY for this wave (only at the ends of its
  // range, or when it holds no rows) are processed as fully masked.
  auto tile_partial = [&](int iter) -> bool {
    if (!wave_active || is_strip(iter) || wave_pad) return true;
    if (SPARSE && wave_code(iter) != 3u) return true;  // one 64-key half only
    const int kt = tile_kt(iter);
    if (it.is_global) return kt * BN + BN > SK;
    return classify_tile(MASK, s.window, SK, wpa, wpb, kt * BN, BN) != TILE_FULL;
  };
  auto tile_empty = [&](int j) -> bool {
    if (!wave_active) return true;
    if (is_strip(j)) return false;
    if (SPARSE && wave_code(j) == 0u) return true;
    return classify_tile(MASK, s.window, SK, wpa, wpb, tile_kt(j) * BN, BN) == TILE_EMPTY;
  };

  // ---- operand reads -------------------------------------------------------
  // K operand (key 32*kbk + l32, dims 16*dc + 8*hf + [0,8)): logical chunk
  // 2*dc + hf, physical (2*dc + hf) ^ ksw(l32) (ksw(32*kbk + l32) = ksw(l32)).
  // The read address of step dc is one lane base XOR (dc << 5): (2*dc + hf)
  // ^ x = 2*(dc ^ (x >> 1)) + (hf ^ (x & 1)) with x = ksw(l32), and 32*(dc ^
  // xh) = 32*dc ^ 32*xh touches bits 5-7 only, which no other term of the
  // address (row, chunk bit 4, a tile base aligned to 1 KiB) does.
  const int k_lane = l32 * ROWB + 16 * (hf ^ (C::ksw(l32) & 1)) + 32 * (C::ksw(l32) >> 1);
  // PERS, wave group 0 from the second item on: Q from the rows its waves
  // staged in LDS during the previous item (same layout and read pattern as
  // the first 32 rows of a K tile).  Only the previous item's 8 stores
  // may have been issued after those direct loads and still be in flight.
  auto load_q_staged = [&]() {
    if constexpr (PERS) {
      static_assert(NDC == 8, "the staged Q read covers eight operands");
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * NDB));
      const unsigned fl = fresh_lane(), fl32 = fl & 31, fhf = fl >> 5;
      const unsigned qb = lds_addr(smem + LDS_MAIN + wave * 32 * ROWB) + fl32 * ROWB +
                          16 * (fhf ^ (C::ksw(fl32) & 1)) + 32 * (C::ksw(fl32) >> 1);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) qf[dc] = lds_read16<0>(qb ^ (unsigned)(dc << 5));
      // (the operands are tied to the wait, so no use is scheduled above it)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]), "+v"(qf[4]), "+v"(qf[5]),
                     "+v"(qf[6]), "+v"(qf[7]));
    }
  };
  auto k_frag = [&](const unsigned char* kbuf, int kbk, int dc) -> bf16x8 {
    const unsigned a = ((lds_addr(kbuf) + k_lane) ^ (unsigned)(dc << 5)) + kbk * 32 * ROWB;
    return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)a;
  };
  // V^T operand (dim 32*db + l32, keys 16*pc + 4*hf + [0,4) then +8) from two
  // ds_read_b64_tr_b16 (v_frags): within each 16-lane group, lane 4t + u addresses the
  // 4 dims 32*db + 16*g + 4u of key 16*pc + 4*hf + t (g = lane bit 4), and the
  // transpose hands lane i element (i & 3) of lanes 4t + (i >> 2), t = 0..3,
  // i.e. dim 32*db + l32 of keys 4*hf + t.  Physical chunk of the 4 dims:
  // (4*db + 2*g + (u >> 1)) ^ (t << VSH), which is 4*(db ^ t) + 2*g + (u >> 1)
  // for VSH = 2 and 4*(db ^ (t >> 1)) + 2*(g ^ (t & 1)) + (u >> 1) for VSH = 1
  // (NDB = 2).  Again the db part is 64*db XORed into bits 6-7 of one lane
  // base, so the read address of block db is (base + v_lane) ^ (db << 6).
  const int tt = (lane >> 2) & 3, uu = lane & 3, gg = (lane >> 4) & 1;
  const int v_lane = (VSH == 2)
                         ? (4 * hf + tt) * ROWB + 64 * tt + 32 * gg + 16 * (uu >> 1) + 8 * (uu & 1)
                         : (4 * hf + tt) * ROWB + 64 * (tt >> 1) + 32 * (gg ^ (tt & 1)) +
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
          const int gk = gpos_s[key < kMaxGlobal ? key : 0];
          const int dist = q_pos - gk;
          // (GEN: padded query rows see nothing, also here)
          const bool vis = key < s.n_global && gk < SK && (dist > s.window || -dist > s.window) &&
                           (!GEN || row_valid);
          sc[kbk][r] = vis ? sc[kbk][r] : -INFINITY;
        }
      return;
    }
    // visible keys of this lane's query as an interval of tile-relative
    // indices, shifted by the lane half so each test is against an immediate:
    // lo <= 32*kbk + 8*(r/4) + r%4 <= hi
    long long lo, hi;
    if (it.is_global) { lo = 0; hi = (long long)SK - 1; }
    else row_interval(MASK, s.window, SK, q_pos, &lo, &hi);
    if (!wave_active || (GEN && !row_valid)) hi = lo - 1;
    const long long base = (long long)tile_kt(iter) * BN + 4 * (PERS ? (int)(fresh_lane() >> 5) : hf);
    const long long tail = (long long)SK - 1;
    const long long hi_a = hi < tail ? hi : tail;
    int lo_r = (int)(lo - base < -1 ? -1 : (lo - base > BN ? BN : lo - base));
    int hi_r = (int)(hi_a - base < -1 ? -1 : (hi_a - base > BN ? BN : hi_a - base));
    if constexpr (SPARSE && BN == 128) {
      // the layout lets this wave see one 64-key half of the tile only
      const unsigned cd = wave_code(iter);
      if (cd == 1u) hi_r = imin(hi_r, 63 - 4 * hf);
      else if (cd == 2u) lo_r = imax(lo_r, 64 - 4 * hf);
    }
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
    const int ntile = cdiv(SK, GK);
    const int t_lo = (int)((long long)ntile * rpart / wph);
    const int t_hi = (int)((long long)ntile * (rpart + 1) / wph);
    const int lrow = lane * 16 / ROWB, lphys = (lane * 16 % ROWB) / 16;
    auto gload = [&](const __bf16* base, int t, unsigned char* dst, bool is_v) {
#pragma unroll
      for (int n = 0; n < NIG; ++n) {
        const int row = n * RPI + lrow;
        const int key = imin(t * GK + row, SKA - 1);  // tail rows repeat a valid row (masked)
        const int sw = is_v ? ((row & 3) << VSH) : C::ksw(row);
        dma16_global((const char*)base + (size_t)key * (is_v ? VRB : KRB) + (lphys ^ sw) * 16,
                     dst + n * 1024);
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
      if ((t + 1) * GK > SK) {
        // tail tile: keys at or beyond SK carry no weight
        const int lim = SK - t * GK - 4 * hf;
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
        for (int db = 0; db < NDB; ++db) vbd[db] = (vb + v_lane) ^ (unsigned)(db << 6);
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
  f32x16 scur[NKB];  // S(j) of this wave's 32 queries
  if constexpr (PERS) {
    // defined on entry to each item: an undefined value carried around the
    // item loop would keep its registers reserved through the whole loop
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
      for (int r = 0; r < 16; ++r) scur[kbk][r] = 0.f;
  }
  bf16x8 pb[NPC];    // P(j), the B operand of O += V(j) P(j); zero where no softmax ran
  auto zero_p = [&]() {
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[pc][t] = (__bf16)0.f;
  };
  zero_p();
  // DBIAS: direct loads issued after this wave's table entries of the last S
  // it computed (its next softmax waits for all but these)
  int bias_after = 0;

  // ---- the matrix block of one step --------------------------------------
  // O^T += V(jv)^T P(jv)^T (if do_pv), then S(js) = K(js) Q^T (if do_s), as
  // straight MFMA sequences whose LDS operands are read up to eight MFMAs
  // ahead.  This wave's direct loads are spread between the MFMAs, so the
  // memory pipe never sees a burst: with four stages, tile dj of K (if dk)
  // or V into stage dst, the same number in every step of a group, which
  // keeps its vmcnt waits exact; with two stages, K(dj) into stage dst and
  // V(dj - 1) into its own stage.  No loads where dj < 0.
  constexpr int NDMA = NSTAGE == 2 ? 2 * NGL : NGL;
  // mode: ModeC<2> (P.V then S), ModeC<0> (P.V only) or ModeC<1> (S only)
  auto mfma_block_m = [&](auto mode, int jv, bool do_pv, int js, bool do_s, bool dk, int dj,
                          int dst) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
    if constexpr (MODE == 0) do_s = false;
    if constexpr (MODE == 1) do_pv = false;
    int dn = 0;
    // the block's two tiles to load: K(dj) (or V(dj) with four stages) and,
    // with two stages, V(dj - 1)
    const TileRsrc t0 = tile_rsrc(dk, dj >= 0 ? dj : 0);
    const TileRsrc t1 = tile_rsrc(false, dj >= 1 ? dj - 1 : 0);
    // the lane bases, opaque per block: the compiler adds each load's row
    // step at the load instead of keeping one offset per load live
    int kl = k_off, vl = v_off;
    asm volatile("" : "+v"(kl), "+v"(vl));
    auto do_dma = [&](int cnt) {
      for (int k = 0; k < cnt; ++k) {
        if (dj >= 0) {
          if (NSTAGE == 2 && dn >= NGL) dma_tile_at(false, t1, (gofs + dj - 1) % NSTAGE, dn - NGL, vl);
          else dma_tile_at(dk, t0, dst, dn, dk ? kl : vl);
        }
        ++dn;
      }
    };
    if (!do_pv && !do_s) {
      do_dma(NDMA);
      return;
    }
    if constexpr (DBIAS) {
      if (do_s) {
        // the table entries of S(js) into this wave's region, before the tile
        // loads of the block: entry t0 + x lands in slot x, where t0 belongs to
        // the tile's first key and the wave's last row.  Entries are clamped
        // into the head's row; only masked pairs ever use a clamped one.
        const int t0 = tile_kt(js) * BN - (wqa + 31 + OFF) + s.Sk - 1;
        const __amdgpu_buffer_rsrc_t br =
            uniform_rsrc(p.bias + (size_t)a * p.bias_len, p.bias_len * 4);
        unsigned char* bdst = smem + LDS_MAIN + LDS_Q + wave * NBD * 256;
#pragma unroll
        for (int n = 0; n < NBD; ++n) {
          const int t = imin(imax(t0 + 64 * n + lane, 0), p.bias_len - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void_t*)(bdst + n * 256), 4, t * 4, 0, 0, 0);
        }
        bias_after = dj >= 0 ? NDMA : 0;
      }
    }
    __builtin_amdgcn_s_setprio(1);
    // One sequence for every block of a mode.  Where P.V is not needed, P is
    // zero (the softmax of that tile was skipped) and its operands are read
    // from the K tile of this block, which has landed (S needs it): a V stage
    // may still be in flight or hold stale bits, and 0 * NaN would not add
    // zero.  Where S is not needed, it is computed from a landed stage and
    // never read.
    const unsigned kb = lds_addr(smem + ((gofs + js) % NSTAGE) * REG);
    const unsigned vb = (MODE == 0 || do_pv) ? lds_addr(smem + NSTAGE * REG + ((gofs + jv) % NSTAGE) * REG) : kb;
    // (the bases are opaque to the compiler, which would otherwise fold the
    // XOR constants into NDB + NDC loop-invariant registers again)
    unsigned v0 = vb + v_lane, k0 = kb + k_lane;
    asm volatile("" : "+v"(v0), "+v"(k0));
    unsigned vbd[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vbd[db] = v0 ^ (unsigned)(db << 6);
    unsigned kbd[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) kbd[dc] = k0 ^ (unsigned)(dc << 5);
    block_run<MODE, ROWB, NDB, NDC, NKB, NDMA>(vbd, kbd, pb, qf, oacc, scur, do_dma);
    __builtin_amdgcn_s_setprio(0);
  };
  auto mfma_block = [&](int jv, bool do_pv, int js, bool do_s, bool dk, int dj,
                        int dst) __attribute__((always_inline)) {
    mfma_block_m(ModeC<2>{}, jv, do_pv, js, do_s, dk, dj, dst);
  };

  // ---- online softmax of S(j): mask, running maximum, weights P(j) and l -----
  auto softmax = [&](int j) __attribute__((always_inline)) {
    if constexpr (DBIAS) {
      // the table entries of S(j) have landed once only the tile loads issued
      // after them may be in flight; register r of block kbk (key 32*kbk +
      // 8*(r/4) + 4*hf + r%4 of the tile) takes slot key + 31 - l32.  Added
      // before the mask, which overwrites every pair it hides.
      if (bias_after == 0) __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
      else __builtin_amdgcn_s_waitcnt(vmcnt_enc(NDMA));
      const float* bl =
          (const float*)(smem + LDS_MAIN + LDS_Q + wave * NBD * 256) + (31 - l32) + 4 * hf;
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          scur[kbk][r] = __builtin_fmaf(bl[kbk * 32 + 8 * (r >> 2) + (r & 3)], p.bias_k, scur[kbk][r]);
    }
    if (tile_partial(j)) {
      asm volatile("");  // keep this a branch: full tiles skip it
      apply_mask(scur, j);
    }
    // ALiBi: minus slope times the distance between key and query positions.
    // Register r of block kbk holds key d0 + 32*kbk + 8*(r/4) + r%4 relative
    // to the query.  Causal masks: every visible key lies at or before the
    // query, so the bias slope*(key - query) is linear in the key; its
    // per-lane part b0 = slope*d0 is carried into the maximum and the
    // exponent instead of into every score.
    float b0 = 0.f;
    if constexpr (ALIBI) {
      const int d0 = tile_kt(j) * BN + 4 * hf - q_pos;
      if constexpr (MASK == MASK_FULL) {
        const float d0f = (float)d0;
#pragma unroll
        for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            scur[kbk][r] = __builtin_fmaf(
                -slope_u, __builtin_fabsf(d0f + (float)(kbk * 32 + 8 * (r >> 2) + (r & 3))),
                scur[kbk][r]);
      } else {
        b0 = slope_u * (float)d0;
#pragma unroll
        for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            scur[kbk][r] =
                __builtin_fmaf((float)(kbk * 32 + 8 * (r >> 2) + (r & 3)), slope_u, scur[kbk][r]);
      }
    }
    float mx;
    {
      // four independent v_max3 chains over the 32 scores of this lane, then join
      float t[2 * NKB];
#pragma unroll
      for (int c4 = 0; c4 < 2 * NKB; ++c4) {
        const int kbk = c4 >> 1, rb = (c4 & 1) * 8;
        float x = max3f(scur[kbk][rb], scur[kbk][rb + 1], scur[kbk][rb + 2]);
        x = max3f(x, scur[kbk][rb + 3], scur[kbk][rb + 4]);
        x = max3f(x, scur[kbk][rb + 5], scur[kbk][rb + 6]);
        t[c4] = max3f(x, scur[kbk][rb + 7], scur[kbk][rb + 7]);
      }
      mx = max3f(max3f(t[0], t[1], t[2]), t[3], t[3]);
#pragma unroll
      for (int c4 = 4; c4 < 2 * NKB; c4 += 2) mx = max3f(mx, t[c4], t[c4 + 1]);
    }
    if constexpr (ALIBI && MASK != MASK_FULL) mx += b0;
    mx = pair_max(mx);
    // rare: a row maximum grew by more than 2^kLazy
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
    float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
    if constexpr (ALIBI && MASK != MASK_FULL) mc -= b0 * c;
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
      const int kbk = pc >> 1, rb = (pc & 1) * 8;
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        bf16x2 pr;
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kbk][rb + t], c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kbk][rb + t + 1], c, -mc));
        pr[0] = (__bf16)e0;
        pr[1] = (__bf16)e1;
        if constexpr (D == 128) {
          // v_dot2 issues to the matrix pipe, which the other wave group keeps
          // busy for a whole D = 128 block: sum the fp32 weights with adds
          if (t & 2) l_run1 += e0 + e1;
          else l_run0 += e0 + e1;
        } else {
          // the denominator sums exactly the rounded weights used in P.V
          if (t & 2) l_run1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run1, false);
          else l_run0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run0, false);
        }
        pb[pc][t] = pr[0];
        pb[pc][t + 1] = pr[1];
      }
    }
  };

  // ---- pipeline ---------------------------------------------------------
  // Tile j lives in stage j % NSTAGE.  The waves form two groups, waves 0-3
  // and 4-7, so that each SIMD runs one wave of each.  Per tile there are two
  // barrier-separated steps; in each, one group runs its matrix block and the
  // other its softmax, so the matrix cores and the vector ALUs of every SIMD
  // work at the same time:
  //   step 2j  : group 0 softmax(S(j)) -> P(j)   | group 1 O += V(j-1)P(j-1); S(j); loads V(j+2)
  //   step 2j+1: group 0 O += V(j)P(j); S(j+1); loads K(j+4) | group 1 softmax(S(j))
  // Loads run two tiles ahead.  K(j) is last read in step 2j, so K(j+4) may
  // overwrite its stage from step 2j+1 on; V(j-2) is last read in step 2j-2,
  // so V(j+2) may overwrite its stage in step 2j.  At the end of step 2j each
  // group waits for its own loads of K(j+1) and V(j) (read from step 2j+1
  // on), letting the two later tiles' loads stay in flight: vmcnt(2*NGL).
  // Every step issues the same number of loads (tiles past the end load a
  // clamped tile), which keeps these counts exact.
  // The steps are separated by bare s_barrier: __syncthreads() adds a
  // workgroup release fence, which the compiler implements by waiting for
  // every direct load in flight.  Direct loads are covered by the explicit
  // vmcnt waits, and every LDS read of a step is waited for before its MFMA.
  // PERS, wave group 0: the Q rows of this wave in item iq into its LDS
  // staging rows by direct loads.  Load n fills
  // rows 4n..4n+3; lane l writes physical chunk l % 16 of row 4n + l / 16,
  // which holds logical chunk (l % 16) ^ ksw(row), the K tile swizzle.  The
  // descriptor covers the item's rows of this wave (rows past the sequence
  // are out of range; their outputs are never stored).
  constexpr int NQL = 32 * ROWB / 1024;  // direct loads per wave
  auto stage_q = [&](const Item& iq) {
    if constexpr (PERS) {
      const unsigned lid = fresh_lane();
      const int qa = iq.blk * s.BMh + rpart * 32;
      const int qb = imin(qa + 31, imin(iq.blk * s.BMh + s.BMh, s.S) - 1);
      const int na = iq.kvh * s.G + iq.hg * s.HP + wave / wph;
      const __amdgpu_buffer_rsrc_t r = uniform_rsrc(
          (const char*)p.q + ((size_t)(iq.b * s.Hq + na) * S + qa) * ROWB,
          qb >= qa ? (qb - qa + 1) * ROWB : 0);
      unsigned char* dst = smem + LDS_MAIN + wave * 32 * ROWB;
#pragma unroll
      for (int n = 0; n < NQL; ++n) {
        const int row = 4 * n + (int)(lid >> 4);
        const int off = row * ROWB + (int)(((lid & 15) ^ (unsigned)C::ksw(row)) * 16);
        dma16_buffer(r, dst + n * 1024, off, 0);
      }
    }
  };
  if constexpr (PERS) {
    static_assert(NSTAGE == 2, "the persistent form runs the two-stage schedule");
    // The schedule below per item, with the loads running on through the
    // stream, the first and last blocks of each group cut to the MFMAs they
    // need (S only, P.V only) and the dead last step dropped: in step 2n
    // group 1 adds its last P.V while group 0 stores its rows; the next item
    // starts with the barrier that ends step 2n, its first K and V tiles
    // already in LDS.  Group 0 loads the tiles in steps 2j+1 (on the first
    // item also the first three), except the last two of the item, K(n+1)
    // and V(n) (the next item's K(1) and V(0)): group 1 loads those in step
    // 2n, so that group 0 stores with no loads in flight, and waits for them
    // before the barrier that ends the next item's step 0.  Group 0 stages
    // the next item's Q in LDS after its first block (its rows there are
    // free once read at the item's start); group 1 loads its Q at the item's
    // start and first needs it in step 0, while group 0 runs S(0) and its
    // softmax.  The vector memory counter retires in order, so group 0's
    // waits for its tile loads leave the Q loads and stores issued after
    // them in flight: nq_out counts those (8 per Q, 8 per set of stores).
    constexpr int NST = 2 * NDB;  // stores per wave (see the epilogue)
    // (each group defines its Q in its own part, so that no path shows the
    // compiler a load into those registers still in flight on the other)
    if (grp == 0) {
      int nq_out = 0;
      if (round == 0) {
        stage_q(it);  // this item's Q, waited for with the first tiles
        int kl = k_off, vl = v_off;
        asm volatile("" : "+v"(kl), "+v"(vl));
        const TileRsrc k0 = tile_rsrc(true, 0), v0 = tile_rsrc(false, 0), k1 = tile_rsrc(true, 1);
        for (int n = 0; n < NGL; ++n) dma_tile_at(true, k0, gofs % NSTAGE, n, kl);
        for (int n = 0; n < NGL; ++n) dma_tile_at(false, v0, gofs % NSTAGE, n, vl);
        for (int n = 0; n < NGL; ++n) dma_tile_at(true, k1, (gofs + 1) % NSTAGE, n, kl);
        __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));  // Q and K(0) landed
      } else {
        nq_out = NST;  // the previous item's stores
      }
      load_q_staged();
      // (later items: K(0) landed before the wait that ended step 2n-2 of
      // the previous item)
      __builtin_amdgcn_s_barrier();
      if (!tile_empty(0)) mfma_block_m(ModeC<1>{}, 0, false, 0, true, true, -1, 0);  // S(0), no loads
      // the wait at the end of step 2j: K(j+1), V(j) landed, the nq_out
      // loads and stores issued after them may still be in flight
      auto wait_tiles = [&]() {
        if (nq_out == 0) __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
        else if (nq_out == NQL) __builtin_amdgcn_s_waitcnt(vmcnt_enc(NQL));
        else if (nq_out == NST) __builtin_amdgcn_s_waitcnt(vmcnt_enc(NST));
        else __builtin_amdgcn_s_waitcnt(vmcnt_enc(NST + NQL));
      };
      for (int j = 0; j < n_it - 1; ++j) {
        if (!tile_empty(j)) softmax(j);  // step 2j
        else zero_p();
        wait_tiles();
        __builtin_amdgcn_s_barrier();
        mfma_block(j, !tile_empty(j), j + 1, !tile_empty(j + 1), true, j + 2, (gofs + j) % NSTAGE);  // step 2j+1
        nq_out = 0;
        // the next item's Q, early: its staging rows are free once read
        if (j == 0 && id_n1 >= 0) {
          stage_q(it_n1);
          nq_out = NQL;
        }
        __builtin_amdgcn_s_barrier();
      }
      if (n_it == 1 && id_n1 >= 0) {
        stage_q(it_n1);
        nq_out += NQL;
      }
      {
        const int j = n_it - 1;
        if (!tile_empty(j)) softmax(j);  // step 2n-2
        else zero_p();
        wait_tiles();
        __builtin_amdgcn_s_barrier();
        mfma_block_m(ModeC<0>{}, j, !tile_empty(j), j, false, true, -1, 0);  // step 2n-1, no loads
        __builtin_amdgcn_s_barrier();
      }
    } else {
      load_q_global();
      __builtin_amdgcn_s_barrier();
      for (int j = 0; j < n_it; ++j) {
        mfma_block(j - 1, j >= 1 && !tile_empty(j - 1), j, !tile_empty(j), false, -1, 0);  // step 2j
        // K(1), V(0), loaded by this group at the end of the previous item,
        // landed before group 0 reads them in step 1
        if (j == 0) __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
        __builtin_amdgcn_s_barrier();
        if (!tile_empty(j)) softmax(j);  // step 2j+1
        else zero_p();
        __builtin_amdgcn_s_barrier();
      }
      // step 2n: the last P.V, with the stream's next two tiles K(n+1) and
      // V(n) (the next item's K(1) and V(0)), whose stages were last read in
      // step 2n-2; this group waits for them before the barrier that ends
      // the next item's step 0
      mfma_block_m(ModeC<0>{}, n_it - 1, !tile_empty(n_it - 1), n_it - 1, false, true, n_it + 1,
                   (gofs + n_it - 1) % NSTAGE);
      // (only those tile loads may be in flight here; the wait tells the
      // compiler so on every path, also where a skipped S(0) never waited
      // for the Q)
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * NGL));
    }
  } else if constexpr (NSTAGE == 2) {
    // Two stages of 128-key tiles (the four-stage schedule below with the
    // loads moved): group 0 loads everything, K(j+2) and V(j+1) in step 2j+1
    // (K(j) and V(j-1) were last read in step 2j: S(j) by group 1, P.V(j-1)
    // by group 1), and waits for all of them at the end of step 2j+2, before
    // the barrier into step 2j+3, the first that reads them.  Group 1 loads
    // nothing, so its waits are implicit in group 0's.
    if (grp == 0) {
      for (int n = 0; n < NGL; ++n) dma(true, 0, 0, n);
      for (int n = 0; n < NGL; ++n) dma(false, 0, 0, n);
      for (int n = 0; n < NGL; ++n) dma(true, 1, 1, n);
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * NGL));  // K(0) landed
    }
    __builtin_amdgcn_s_barrier();
    if (grp == 0) {
      if (!tile_empty(0)) mfma_block(0, false, 0, true, true, -1, 0);  // S(0), no loads
      for (int j = 0; j <= n_it; ++j) {
        if (j < n_it && !tile_empty(j)) softmax(j);  // step 2j
        else zero_p();
        __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));  // K(j+1), V(j) landed
        __builtin_amdgcn_s_barrier();
        mfma_block(j, j < n_it && !tile_empty(j), j + 1, j + 1 < n_it && !tile_empty(j + 1),
                   true, j + 2, j % NSTAGE);  // step 2j+1
        __builtin_amdgcn_s_barrier();
      }
    } else {
      for (int j = 0; j <= n_it; ++j) {
        mfma_block(j - 1, j >= 1 && !tile_empty(j - 1), j, j < n_it && !tile_empty(j),
                   false, -1, 0);  // step 2j
        __builtin_amdgcn_s_barrier();
        if (j < n_it && !tile_empty(j)) softmax(j);  // step 2j+1
        else zero_p();
        __builtin_amdgcn_s_barrier();
      }
    }
  } else {
  if (grp == 0) {
    for (int n = 0; n < NGL; ++n) dma(true, 0, 0, n);
    for (int n = 0; n < NGL; ++n) dma(true, 1, 1, n);
    for (int n = 0; n < NGL; ++n) dma(true, 2, 2, n);
    for (int n = 0; n < NGL; ++n) dma(true, 3, 3, n);
    __builtin_amdgcn_s_waitcnt(0x0f70 | (3 * NGL));  // K(0) landed
  } else {
    for (int n = 0; n < NGL; ++n) dma(false, 0, 0, n);
    for (int n = 0; n < NGL; ++n) dma(false, 1, 1, n);
  }
  __builtin_amdgcn_s_barrier();

  if (grp == 0) {
    if (!tile_empty(0)) mfma_block(0, false, 0, true, true, -1, 0);  // S(0), no loads
    for (int j = 0; j <= n_it; ++j) {
      if (j < n_it && !tile_empty(j)) softmax(j);  // step 2j
      else zero_p();
      __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NGL));  // K(j+1) landed
      __builtin_amdgcn_s_barrier();
      mfma_block(j, j < n_it && !tile_empty(j), j + 1, j + 1 < n_it && !tile_empty(j + 1),
                 true, j + 4, (j + 4) % NSTAGE);  // step 2j+1
      __builtin_amdgcn_s_barrier();
    }
  } else {
    for (int j = 0; j <= n_it; ++j) {
      mfma_block(j - 1, j >= 1 && !tile_empty(j - 1), j, j < n_it && !tile_empty(j),
                 false, j + 2, (j + 2) % NSTAGE);  // step 2j
      __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NGL));  // V(j) landed
      __builtin_amdgcn_s_barrier();
      if (j < n_it && !tile_empty(j)) softmax(j);  // step 2j+1
      else zero_p();
      __builtin_amdgcn_s_barrier();
    }
  }
  }
  // no direct load may land after the workgroup ends (PERS: after its last
  // item; the loads in flight between items belong to the next one)
  if constexpr (!PERS) __builtin_amdgcn_s_waitcnt(0x0f70);
  }  // ping-pong path

  // ---- PERS: this item's O --------------------------------------------------
  // Stores through a scalar descriptor over the wave's rows and a lane offset
  // from a freshly read lane id, so nothing long-lived is needed here.
  if constexpr (PERS) {
    const unsigned lid = fresh_lane();
    const int row_off = (int)(lid & 31) * ROWB;
    const unsigned lu = __float_as_uint(l_run0 + l_run1);
    const auto sw = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
    const float inv = 1.f / (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
    const int qa = r0 + rpart * 32;
    const __amdgpu_buffer_rsrc_t r = uniform_rsrc(
        (char*)p.o + ((size_t)(it.b * s.Hq + a) * S + qa) * ROWB,
        wave_active ? (wqb - qa + 1) * ROWB : 0);
    // Lane (row, h) holds dims 32*db + 8*g4 + 4*h + [0, 4) of its row.  For
    // each pair g4 = 2*g2, 2*g2 + 1 one swap between the lane halves gives
    // lane h the 8 dims 32*db + 16*g2 + 8*h + [0, 8): 16 bytes per store,
    // 32 contiguous bytes of each row per instruction.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        bf16x4 wa, wb;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          wa[t] = (__bf16)(oacc[db][(2 * g2) * 4 + t] * inv);
          wb[t] = (__bf16)(oacc[db][(2 * g2 + 1) * 4 + t] * inv);
        }
        const u32x2 a2 = __builtin_bit_cast(u32x2, wa), b2 = __builtin_bit_cast(u32x2, wb);
        // swap(a, b): lanes 0-31 get (a, a of lane + 32), lanes 32-63 (b of lane - 32, b)
        const auto s0 = __builtin_amdgcn_permlane32_swap(a2[0], b2[0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a2[1], b2[1], false, false);
        const u32x4 c = {s0[0], s1[0], s0[1], s1[1]};
        __builtin_amdgcn_raw_buffer_store_b128(c, r, row_off + (db * 32 + g2 * 16) * 2 + (int)(lid >> 5) * 16,
                                               0, 0);
      }
  } else
  // ---- epilogue: O = O^T / l, round to bf16, store --------------------------
  {
    const float l_run = l_run0 + l_run1;
    const unsigned lu = __float_as_uint(l_run);
    const float l_other = __uint_as_float(__shfl_xor((int)lu, 32));
    const float l_tot = l_run + l_other;
    // global items: the first wave of each head holds the merged result
    // (GEN: padded query rows and rows that see no key are written as zero)
    bool store = it.is_global ? row_valid && rpart == 0
                              : (GEN ? q_row < s.S : row_valid && wave_active);
    // band items leave the rows of global queries to the global items (GEN:
    // padded rows, which no global item owns, are still written as zero)
    if (MASK == MASK_LOCAL_GLOBAL && !it.is_global && store && (!GEN || q_row < SQ)) {
      for (int g = 0; g < s.n_global; ++g) store = store && (gpos_s[g] != q_pos);
    }
    if (store) {
      const float inv = GEN ? (l_tot > 0.f ? 1.f / l_tot : 0.f) : 1.f / l_tot;
      __bf16* op = GEN ? (__bf16*)p.o + it.b * p.os[0] + a * p.os[1] + q_row * p.os[2]
                       : (__bf16*)p.o + ((size_t)(it.b * s.Hq + a) * S + q_row) * D;
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
  gofs += n_it;
  }  // items
  if constexpr (PERS) __builtin_amdgcn_s_waitcnt(0x0f70);
}

template <int D>
hipError_t launch_d(const KParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.s.n_items), block(kBf16Threads);
  if (p.general && p.layout) {
    const bool full = p.s.mask == MASK_FULL;
    if (p.s.S <= kSparseShortKeys) {
      if (full) hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_FULL, 3>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL, 3>), grid, block, 0, stream, p);
    } else {
      if (full) hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_FULL, 5>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL, 5>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
  }
  if (p.general && p.bias) {
    switch (p.s.mask) {
      case MASK_FULL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_FULL, 4>), grid, block, 0, stream, p); break;
      case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL, 4>), grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL_WINDOW, 4>), grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
  }
  if (p.general && p.slopes) {
    switch (p.s.mask) {
      case MASK_FULL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_FULL, 2>), grid, block, 0, stream, p); break;
      case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL, 2>), grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL_WINDOW, 2>), grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
  }
  if (p.general) {
    switch (p.s.mask) {
      case MASK_FULL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_FULL, 1>), grid, block, 0, stream, p); break;
      case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL, 1>), grid, block, 0, stream, p); break;
      case MASK_CAUSAL_WINDOW: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL_WINDOW, 1>), grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_LOCAL_GLOBAL, 1>), grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
  }
  switch (p.s.mask) {
    case MASK_FULL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_FULL>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL>), grid, block, 0, stream, p); break;
    case MASK_CAUSAL_WINDOW: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_CAUSAL_WINDOW>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((attn_fwd_bf16<D, MASK_LOCAL_GLOBAL>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

#if ATTN_HEAD_DIM == 128
hipError_t launch_bf16_pers_d128(const KParams& p, int grid, hipStream_t stream) {
  dim3 g((unsigned)grid), block(kBf16Threads);
  switch (p.s.mask) {
    case MASK_FULL: hipLaunchKernelGGL((attn_fwd_bf16<128, MASK_FULL, 0, 1>), g, block, 0, stream, p); break;
    case MASK_CAUSAL: hipLaunchKernelGGL((attn_fwd_bf16<128, MASK_CAUSAL, 0, 1>), g, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((attn_fwd_bf16<128, MASK_CAUSAL_WINDOW, 0, 1>), g, block, 0, stream, p); break;
  }
  return hipGetLastError();
}
#endif

#if ATTN_HEAD_DIM == 64
hipError_t launch_bf16_d64(const KParams& p, hipStream_t stream) { return launch_d<64>(p, stream); }
#else
hipError_t launch_bf16_d128(const KParams& p, hipStream_t stream) { return launch_d<128>(p, stream); }
#endif

}  // namespace attn
