// kernel_decode.hip -- bf16 decode attention against a key/value cache on gfx950.
//
// Method: the Sq newest positions of each sequence attend to the cached keys
// and values of that sequence ("Trasformer 浅析", section 推理：KV 缓存: the
// step-t output is the softmax of q_t against the cached keys of positions
// 1..t, applied to the cached values; "Transformer 架构及其变体", section
// 预填充创建缓存，解码复用缓存: decode reads the whole retained cache each
// step, so it is bound by memory bandwidth, and the sequences of a batch hold
// caches of different lengths).  Query i of the Sq new ones sits at cache
// position L - Sq + i; the causal mask lets it see positions 0..L - Sq + i,
// the full mask all L.  Under a sliding window of w positions ("Transformer
// 演进与变体", section 稀疏注意力: each position attends to the w positions
// up to itself) query i sees L - Sq + i - w < j <= L - Sq + i, so a sequence
// reads only its last w + Sq - 1 positions.
//
// gfx950 mapping:
//   * One workgroup of eight wave64 per (sequence b, key/value head, key
//     split).  The 32 query columns of v_mfma_f32_32x32x16_bf16 hold the
//     G * Sq query rows of the group (G = Hq / Hkv heads x Sq positions, at
//     most 32), so every cached key and value row is read from HBM once for
//     all query heads that share it ("第 8 章 AI 算法Transformer大模型",
//     section 8.2.1: shared key/value heads need one read instead of h).
//   * Splits: a sequence's key range is cut into runs of at most `per`
//     32-key tiles, with per as small as the rule "all work items fit in one
//     wave of 256 workgroups (one per CU)" allows, so a long sequence takes
//     more splits than a short one and no split is empty.  With the lengths
//     on the device every workgroup derives the same plan from them (a
//     search for per, then a scan that finds its (b, split)); without, all
//     sequences are alike and the plan is the host's.
//   * The split's keys are cut into 32-key tiles; wave w walks tiles w,
//     w + 8, ... (so the eight waves stream neighbouring tiles of one
//     contiguous range at any time) through a private LDS region (one K
//     tile and one V tile, loaded straight into LDS), so the walk needs no
//     workgroup barrier: the next K tile loads while the softmax of the
//     current one runs, the next V tile while its P.V runs.  Operands: K with ds_read_b128, V^T with
//     ds_read_b64_tr_b16, both under the swizzles of the prefill kernel.
//   * Online softmax per wave in log2 units with lazy rescaling, then the
//     waves' partial (m, l, O) merge through LDS in a fixed pairing order.
//   * One split: O / l is written as bf16.  Several splits: the partial
//     (m, l, O) goes to the caller's workspace and the combine kernel merges
//     the splits of each row with the same recurrence (one workgroup per
//     row, four thread groups over the splits).
//   * A plain streaming read of 1 GiB reaches about 6.0-6.3 TB/s on MI355X
//     (LDS-direct or vector loads); that, not the 8 TB/s peak, is the
//     practical ceiling of this kernel.
#include "attn_decode.h"
#include "gfx950_ops.h"

namespace attn {
namespace {

constexpr int DT = 32;              // keys per tile
constexpr int DWAVES = 8;           // waves per workgroup
constexpr float kDLazy = 8.f;       // rescale threshold, log2 units

template <int D>
struct DCfg {
  static constexpr int NDC = D / 16;           // 16-dim reduction steps of S^T
  static constexpr int NDB = D / 32;           // 32-dim blocks of O^T
  static constexpr int ROWB = D * 2;           // bytes per K or V row
  static constexpr int REG = DT * ROWB;        // one private K or V tile
  static constexpr int NIG = REG / 1024;       // 1 KiB direct loads per tile
  static constexpr int RPI = 1024 / ROWB;      // tile rows per 1 KiB load
  static constexpr int VSH = D == 128 ? 2 : 1; // V chunk swizzle shift
  static __device__ constexpr int ksw(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  static constexpr int SLOT = 4 * NDB * 64 * 16 + 64 * 8;  // one wave's partial for the merge
  static constexpr int LDS = DWAVES * 2 * REG;
  static_assert(DWAVES / 2 * SLOT <= LDS, "merge slots fit in the walk regions");
  static_assert(NIG < 16, "vmcnt immediates below 16");
};

// Length of sequence b (lengths outside [0, Smax] are clamped).
__device__ __forceinline__ int decode_len(const DParams& p, int b) {
  const int L = p.cache_len[b];
  return L < 0 ? 0 : (L > p.Smax ? p.Smax : L);
}
// Inclusive prefix sum (ADD) or prefix maximum of non-negative values over
// the 64 lanes of a wave with DPP row moves (a few cycles each, no LDS):
// shifts by 1, 2, 4 and 8 within each row of 16 lanes, then the last lane of
// row 0 into row 1 and of row 2 into row 3, then the last lane of row 1 into
// rows 2 and 3.  Lanes without a source read 0.
template <bool ADD, typename T>
__device__ __forceinline__ T wave_scan(T x) {
  auto op = [](T a, T b) { return ADD ? a + b : (a > b ? a : b); };
  x = op(x, __builtin_amdgcn_update_dpp((T)0, x, 0x111, 0xf, 0xf, true));  // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp((T)0, x, 0x112, 0xf, 0xf, true));  // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp((T)0, x, 0x114, 0xf, 0xf, true));  // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp((T)0, x, 0x118, 0xf, 0xf, true));  // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp((T)0, x, 0x142, 0xa, 0xf, false)); // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp((T)0, x, 0x143, 0xc, 0xf, false)); // row_bcast:31
  return x;
}
// the scan's value in lane 63: the wave's total or maximum
template <bool ADD, typename T>
__device__ __forceinline__ T wave_all(T x) {
  x = wave_scan<ADD>(x);
  if constexpr (sizeof(T) == 8) {
    const unsigned lo = __builtin_amdgcn_readlane((unsigned)x, 63);
    const unsigned hi = __builtin_amdgcn_readlane((unsigned)((unsigned long long)x >> 32), 63);
    return (T)(((unsigned long long)hi << 32) | lo);
  } else {
    return __builtin_amdgcn_readlane(x, 63);
  }
}

template <int D>
__global__ __launch_bounds__(DWAVES * 64) void attn_decode_bf16(DParams p) {
  using C = DCfg<D>;
  constexpr int NDC = C::NDC, NDB = C::NDB, ROWB = C::ROWB, REG = C::REG, NIG = C::NIG,
                RPI = C::RPI, VSH = C::VSH, SLOT = C::SLOT;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // ---- work item: (b, kvh, split) ---------------------------------------------
  int b, kvh, split, ns, slot, Lf;
  if (p.uni_splits) {
    // every sequence holds Smax positions: the host's split count
    ns = p.uni_splits;
    const int pair = (int)blockIdx.x / ns;
    split = (int)blockIdx.x % ns;
    b = pair / p.Hkv;
    kvh = pair % p.Hkv;
    slot = pair * ns;
    Lf = p.Smax;
  } else {
    // The same plan in every wave of every workgroup, from the lengths (no
    // LDS, no barrier): a split holds at most `per` tiles, per the smallest
    // value found for which the items, Hkv * sum_b ceil(tiles_b / per), fit
    // in kDecodeWorkgroups (one wave of workgroups); then item g is split
    // g - Hkv * (s_0 + .. + s_{b-1}) of sequence b, in (kvh, split) order,
    // and only pairs with two or more splits take partial slots.  Lanes hold
    // sequences lane, lane + 64, ...; the first 64 lengths stay in a register.
    const int nch = (p.B + 63) / 64;
    const int L0 = lane < p.B ? decode_len(p, lane) : 0;
    auto len_at = [&](int ch) {
      const int bb = ch * 64 + lane;
      return ch == 0 ? L0 : (bb < p.B ? decode_len(p, bb) : 0);
    };
    auto tiles_of = [&](int L) { return (L - decode_first_key(L, p.Sq, p.window) + DT - 1) / DT; };
    // items of the plan with at most `per` tiles per split
    auto items = [&](int per) {
      long long n = 0;
      for (int ch = 0; ch < nch; ++ch)
        if (ch * 64 + lane < p.B) n += decode_splits(tiles_of(len_at(ch)), per);
      return wave_all<true>(n) * p.Hkv;
    };
    long long ts = 0;
    int tm = 0;
    for (int ch = 0; ch < nch; ++ch) {
      const int t = tiles_of(len_at(ch));
      ts += t;
      tm = t > tm ? t : tm;
    }
    const long long T = wave_all<true>(ts);
    const int TM = wave_all<false>(tm);
    const int K = kDecodeWorkgroups / p.Hkv;  // splits per key/value head
    int per;
    if (K <= p.B || T == 0) {
      per = TM > kDecodeMinTiles ? TM : kDecodeMinTiles;  // one split each
    } else {
      // lower bound: Hkv * T / per items at least
      const long long lo0 = (T * p.Hkv + kDecodeWorkgroups - 1) / kDecodeWorkgroups;
      int lo = lo0 > kDecodeMinTiles ? (int)lo0 : kDecodeMinTiles;
      if (items(lo) <= kDecodeWorkgroups) {
        per = lo;
      } else {
        // upper bound: the proportional plan 1 + floor((K - B) tiles_b / T)
        // holds at most K splits per head, its largest split `hi` tiles, and
        // ceil(tiles_b / hi) never exceeds its split count
        int hi = kDecodeMinTiles;
        for (int ch = 0; ch < nch; ++ch) {
          const int t = tiles_of(len_at(ch));
          const int sb = 1 + (int)((long long)(K - p.B) * t / T);
          const int h = (t + sb - 1) / sb;
          hi = h > hi ? h : hi;
        }
        hi = wave_all<false>(hi);
        hi = hi > lo ? hi : lo + 1;
        // lo fails, hi fits: bisect, at most six steps (to a 64th of the
        // first interval)
        for (int step = 0; step < 6 && hi - lo > 1; ++step) {
          const int mid = lo + (hi - lo) / 2;
          if (items(mid) <= kDecodeWorkgroups) hi = mid;
          else lo = mid;
        }
        per = hi;
      }
    }
    // scan the split counts for the sequence that holds item g
    const int g = (int)blockIdx.x;
    int carry_s = 0, carry_q = 0, fb = -1, fs = 0, fe = 0, fq = 0, fl = 0;
    for (int ch = 0; ch < nch; ++ch) {
      const int bb = ch * 64 + lane;
      const int Lb = len_at(ch);
      const int sb = bb < p.B ? decode_splits(tiles_of(Lb), per) : 0;
      const int qb = sb >= 2 ? sb : 0;
      const int is = wave_scan<true>(sb), iq = wave_scan<true>(qb);  // inclusive
      const int first = p.Hkv * (carry_s + is - sb);
      const unsigned long long hit =
          __builtin_amdgcn_ballot_w64(bb < p.B && g >= first && g < first + p.Hkv * sb);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        fb = ch * 64 + src;
        fs = __builtin_amdgcn_readlane(sb, src);
        fe = g - __builtin_amdgcn_readlane(first, src);
        fq = carry_q + __builtin_amdgcn_readlane(iq - qb, src);
        fl = __builtin_amdgcn_readlane(Lb, src);
        break;
      }
      carry_s += __builtin_amdgcn_readlane(is, 63);
      carry_q += __builtin_amdgcn_readlane(iq, 63);
    }
    if (fb < 0) return;  // past the last item (the grid is an upper bound)
    b = fb;
    ns = fs;
    kvh = fe / ns;
    split = fe % ns;
    slot = p.Hkv * fq + kvh * ns;
    Lf = fl;
  }
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  split = __builtin_amdgcn_readfirstlane(split);
  ns = __builtin_amdgcn_readfirstlane(ns);
  slot = __builtin_amdgcn_readfirstlane(slot);
  // a plan whose partials would not fit the workspace is never carried out
  if (ns >= 2 && (!p.ws || slot + ns > p.max_slots)) return;
  const int L = __builtin_amdgcn_readfirstlane(Lf);
  const int kfirst = decode_first_key(L, p.Sq, p.window);

  // ---- this lane's query row: head kvh*G + r / Sq, new position r % Sq ----------
  const int r = l32;
  const int nrows = p.G * p.Sq;
  const bool row_valid = r < nrows;
  const int a = kvh * p.G + (row_valid ? r / p.Sq : 0);
  const int qi = row_valid ? r % p.Sq : 0;
  // last visible cache position of this row (inclusive); -1 when it sees none
  const int lim = p.causal ? L - p.Sq + qi : L - 1;
  // window: this row sees positions lim - w + 1 .. lim

  const size_t Smax = (size_t)p.Smax;
  const __bf16* kp = (const __bf16*)p.k + ((size_t)b * p.Hkv + kvh) * Smax * D;
  const __bf16* vp = (const __bf16*)p.v + ((size_t)b * p.Hkv + kvh) * Smax * D;

  // ---- Q^T operand: lane holds row r, dims 16*dc + 8*hf + [0, 8) ---------------
  bf16x8 qf[NDC];
  {
    const __bf16* qrow = (const __bf16*)p.q + (((size_t)b * p.Hq + a) * p.Sq + qi) * D;
    const u32x4 flip = (p.qmode == 1) ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                                      : u32x4{0u, 0u, 0u, 0u};
    const bool zero = (p.qmode == 2) || !row_valid;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (!zero) x = *(const u32x4*)(qrow + dc * 16 + hf * 8);
      x ^= flip;
      qf[dc] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- the split's key range [k0, k1) in 32-key tiles -------------------------
  // the sequence's tiles from kfirst, cut into ns runs of equal length (the
  // last one shorter); every run starts before L
  const int seq_tiles = (L - kfirst + DT - 1) / DT;
  const int tps = (seq_tiles + ns - 1) / ns;
  const int k0 = kfirst + split * tps * DT;
  const int k1 = (tps * DT < L - k0) ? k0 + tps * DT : L;
  const int ntile = k1 > k0 ? (k1 - k0 + DT - 1) / DT : 0;

  unsigned char* kreg = smem + wave * 2 * REG;
  unsigned char* vreg = kreg + REG;
  // Direct load of tile t (keys k0 + 32 t ..): lane l fills 16 bytes of row
  // n * RPI + l * 16 / ROWB.  Rows at or past L repeat the last valid row (their
  // scores are masked, so they carry zero weight, and stay finite).
  const int lrow = lane * 16 / ROWB, lphys = (lane * 16 % ROWB) / 16;
  auto gload = [&](const __bf16* base, int t, unsigned char* dst, bool is_v) {
#pragma unroll
    for (int n = 0; n < NIG; ++n) {
      const int row = n * RPI + lrow;
      const int key = imin(k0 + t * DT + row, L - 1);
      const int sw = is_v ? ((row & 3) << VSH) : C::ksw(row);
      dma16_global((const char*)base + (size_t)key * ROWB + (lphys ^ sw) * 16, dst + n * 1024);
    }
  };

  // operand read bases (same layouts as the prefill kernel)
  int k_rd[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) k_rd[dc] = l32 * ROWB + 16 * ((2 * dc + hf) ^ C::ksw(l32));
  const int tt = (lane >> 2) & 3, uu = lane & 3, gg = (lane >> 4) & 1;
  int v_rd[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    v_rd[db] = (VSH == 2)
                   ? (4 * hf + tt) * ROWB + 64 * (db ^ tt) + 32 * gg + 16 * (uu >> 1) + 8 * (uu & 1)
                   : (4 * hf + tt) * ROWB + 64 * (db ^ (tt >> 1)) + 32 * (gg ^ (tt & 1)) +
                         16 * (uu >> 1) + 8 * (uu & 1);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q = 0; q < 16; ++q) oacc[db][q] = 0.f;
  float m_run = -INFINITY, l_run0 = 0.f, l_run1 = 0.f;
  const float c = p.c;
  // keys past lim_lo or before lo_hi are masked for some row of the wave
  const int lim_lo = p.causal ? L - p.Sq : L - 1;
  const int lo_hi = p.window ? L - p.window : -(1 << 30);
  // first position this row sees (0 without a window; no key loaded is below it
  // then)
  const int row_lo = (p.window && lim - p.window + 1 > 0) ? lim - p.window + 1 : 0;

  // wave w takes tiles w, w + 8, ...: at any time the eight waves stream
  // neighbouring tiles of one contiguous range
  if (wave < ntile) {
    gload(kp, wave, kreg, false);
    gload(vp, wave, vreg, true);
  }
  for (int t = wave; t < ntile; t += DWAVES) {
    const bool more = t + DWAVES < ntile;
    __builtin_amdgcn_s_waitcnt(0x0f70 | NIG);  // K(t) landed; V(t) may be in flight
    f32x16 sc;
#pragma unroll
    for (int q = 0; q < 16; ++q) sc[q] = 0.f;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) sc = mfma32(*(const bf16x8*)(kreg + k_rd[dc]), qf[dc], sc);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // K operand reads done: the region may be refilled
    if (more) gload(kp, t + DWAVES, kreg, false);
    const int tk = k0 + t * DT;
    if (tk + DT - 1 > lim_lo || tk < lo_hi) {
      // register q of the accumulator holds key tk + 8*(q/4) + 4*hf + q%4; the
      // row sees offsets rel - w + 1 .. rel
      const int rel = lim - tk - 4 * hf;
      const int rlo = row_lo - tk - 4 * hf;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int off = 8 * (q >> 2) + (q & 3);
        sc[q] = (off <= rel && off >= rlo) ? sc[q] : -INFINITY;
      }
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
    if (__builtin_amdgcn_ballot_w64(mx * c > m_run * c + kDLazy) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);
      m_run = m_new;
      l_run0 *= alpha;
      l_run1 *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q = 0; q < 16; ++q) oacc[db][q] *= alpha;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
    bf16x8 pb[2];
#pragma unroll
    for (int pc = 0; pc < 2; ++pc)
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * pc + u], c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * pc + u + 1], c, -mc));
        if (u & 2) l_run1 += e0 + e1;
        else l_run0 += e0 + e1;
        pb[pc][u] = (__bf16)e0;
        pb[pc][u + 1] = (__bf16)e1;
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
    if (more) gload(vp, t + DWAVES, vreg, true);
  }

  // ---- merge the eight waves' partial (m, l, O): chunk w takes chunk w + half --
  // In the O^T accumulator lane l of every wave owns the same (row, dims), so
  // partials combine lane by lane:
  //   m = max(m1, m2),  X = X1 * 2^((m1 - m) c) + X2 * 2^((m2 - m) c)  for X in {l, O}.
  for (int half = DWAVES / 2; half >= 1; half >>= 1) {
    __syncthreads();  // the walk regions (first pass) or slots (later passes) are free
    if (wave >= half && wave < 2 * half) {
      unsigned char* sl = smem + (wave - half) * SLOT;
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
    if (wave < half) {
      const unsigned char* sl = smem + wave * SLOT;
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
  if (wave != 0) return;

  // ---- wave 0: the workgroup's (m, l, O) of the 32 rows ---------------------------
  const float l_half = l_run0 + l_run1;
  const float l_tot = l_half + __uint_as_float(__shfl_xor((int)__float_as_uint(l_half), 32));
  if (p.ws && !p.uni_splits && split == 0 && lane == 0)
    *(int2*)(p.hdr + 2 * (b * p.Hkv + kvh)) = int2{slot, ns};
  if (ns == 1) {
    if (!row_valid) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;  // a row that sees nothing is zero
    __bf16* op = (__bf16*)p.o + (((size_t)b * p.Hq + a) * p.Sq + qi) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (__bf16)(oacc[db][g4 * 4 + q] * inv);
        *(bf16x4*)(op + db * 32 + g4 * 8 + hf * 4) = w;
      }
    return;
  }
  // partial of this split: rows [32][D] fp32 (unnormalised O), then m (log2
  // units, -inf when the row saw nothing here) and l per row
  float* ws = p.ws + (size_t)(slot + split) * (32 * (D + 2));
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 x = {oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2],
                        oacc[db][4 * g4 + 3]};
      *(float4*)(ws + r * D + db * 32 + g4 * 8 + hf * 4) = x;
    }
  if (hf == 0) {
    ws[32 * D + r] = m_run == -INFINITY ? -INFINITY : m_run * c;
    ws[32 * D + 32 + r] = l_tot;
  }
}

// Merge the splits of one query row: one workgroup of 512 threads per (b,
// kvh, row) (pairs that took one split wrote their output already).  Thread
// (g, c) holds dims 4c .. 4c + 3 and walks the splits s = g mod CG with the
// online recurrence (running maximum M; numerator and denominator rescaled by
// 2^(M_old - M_new) when it rises), so every partial is read once; the CG
// groups then meet in LDS in a fixed order:
//   M = max_s m_s,  O[d] = sum_s 2^(m_s - M) O_s[d] / sum_s 2^(m_s - M) l_s
// (zero when no split saw a position).
constexpr int kCombThreads = 512;
template <int D>
__global__ __launch_bounds__(kCombThreads) void attn_decode_combine(DParams p) {
  constexpr int STRIDE = 32 * (D + 2);
  constexpr int TPR = D / 4;                 // threads per row
  constexpr int CG = kCombThreads / TPR;     // split groups
  __shared__ float4 pnum[CG][TPR];
  __shared__ float2 pmd[CG];
  const int nrows = p.G * p.Sq;
  const int pair = (int)blockIdx.x / nrows, r = (int)blockIdx.x % nrows;
  const int b = pair / p.Hkv, kvh = pair % p.Hkv;
  const int tid = threadIdx.x, c = tid % TPR, g = tid / TPR;
  int ns = p.uni_splits, slot = pair * ns;
  if (!ns) {
    const int2 h = *(const int2*)(p.hdr + 2 * pair);
    slot = h.x;
    ns = h.y;
  }
  if (ns < 2 || slot + ns > p.max_slots) return;
  const float* base = p.ws + (size_t)slot * STRIDE;
  float M = -INFINITY, den = 0.f;
  float4 num = {0.f, 0.f, 0.f, 0.f};
  // four of the thread's splits per round, all loads issued before any use
  constexpr int U = 4;
  for (int s0 = g; s0 < ns; s0 += U * CG) {
    float ms[U], ls[U];
    float4 os[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + u * CG;
      ms[u] = -INFINITY;
      ls[u] = 0.f;
      os[u] = float4{0.f, 0.f, 0.f, 0.f};
      if (sp < ns) {
        const float* w = base + (size_t)sp * STRIDE;
        ms[u] = w[32 * D + r];
        ls[u] = w[32 * D + 32 + r];
        os[u] = *(const float4*)(w + r * D + 4 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ms[u] == -INFINITY) continue;  // the split saw no position of the row
      if (ms[u] > M) {
        const float f = __builtin_amdgcn_exp2f(M - ms[u]);  // 0 while M is -inf
        den *= f;
        num.x *= f;
        num.y *= f;
        num.z *= f;
        num.w *= f;
        M = ms[u];
      }
      const float f = __builtin_amdgcn_exp2f(ms[u] - M);
      den += f * ls[u];
      num.x += f * os[u].x;
      num.y += f * os[u].y;
      num.z += f * os[u].z;
      num.w += f * os[u].w;
    }
  }
  pnum[g][c] = num;
  if (c == 0) pmd[g] = float2{M, den};
  __syncthreads();
  if (g != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int k = 0; k < CG; ++k) Mt = fmaxf(Mt, pmd[k].x);
  float4 o = {0.f, 0.f, 0.f, 0.f};
  if (Mt != -INFINITY) {
    float dt = 0.f;
    float4 nt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < CG; ++k) {
      const float2 md = pmd[k];
      if (md.x == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(md.x - Mt);
      const float4 x = pnum[k][c];
      dt += f * md.y;
      nt.x += f * x.x;
      nt.y += f * x.y;
      nt.z += f * x.z;
      nt.w += f * x.w;
    }
    if (dt > 0.f) {
      const float inv = 1.f / dt;
      o = float4{nt.x * inv, nt.y * inv, nt.z * inv, nt.w * inv};
    }
  }
  const int a = kvh * p.G + r / p.Sq, qi = r % p.Sq;
  bf16x4 w4;
  w4[0] = (__bf16)o.x;
  w4[1] = (__bf16)o.y;
  w4[2] = (__bf16)o.z;
  w4[3] = (__bf16)o.w;
  *(bf16x4*)((__bf16*)p.o + (((size_t)b * p.Hq + a) * p.Sq + qi) * D + 4 * c) = w4;
}

template <int D>
hipError_t launch_decode_d(const DParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(attn_decode_bf16<D>, dim3((unsigned)grid), dim3(DWAVES * 64), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !p.ws) return err;
  const long long rows = (long long)p.B * p.Hkv * p.G * p.Sq;
  hipLaunchKernelGGL(attn_decode_combine<D>, dim3((unsigned)rows), dim3(kCombThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DParams& p, int D, int grid, hipStream_t stream) {
  return D == 64 ? launch_decode_d<64>(p, grid, stream) : launch_decode_d<128>(p, grid, stream);
}

}  // namespace attn
