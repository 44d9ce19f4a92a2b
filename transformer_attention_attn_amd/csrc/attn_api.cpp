// attn_api.cpp -- the C ABI of libattn.so: argument validation, normalisation
// of the global-token set, work planning and kernel dispatch.  No device
// memory is allocated; all launch data travels in the kernel argument block.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/attn.h"
#include "attn_decode.h"
#include "attn_kernels.h"

namespace {

using attn::KParams;
using attn::Sched;

constexpr int kVersion = 200;  // 0.2.0
constexpr long long kMaxS = 1LL << 30;

struct Checked {
  int status;
  Sched s;
  int gpos[attn::kMaxGlobal];
  int n_global;  // distinct
};

Checked check_args(int B, int Hq, int Hkv, int S, int D, int mask_kind, int window,
                   const int* global_idx, int n_global, int dtype) {
  Checked c{};
  c.status = ATTN_OK;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || (long long)S > kMaxS) { c.status = ATTN_ERR_SHAPE; return c; }
  const bool fp8 = dtype == ATTN_DTYPE_FP8_E4M3 || dtype == ATTN_DTYPE_FP8_E5M2;
  if (dtype != ATTN_DTYPE_FP32 && dtype != ATTN_DTYPE_BF16 && !fp8) {
    c.status = ATTN_ERR_UNSUPPORTED;
    return c;
  }
  if (D != 64 && D != 128) { c.status = ATTN_ERR_UNSUPPORTED; return c; }
  if (mask_kind < ATTN_MASK_FULL || mask_kind > ATTN_MASK_LOCAL_GLOBAL) { c.status = ATTN_ERR_UNSUPPORTED; return c; }
  if (Hq % Hkv != 0) { c.status = ATTN_ERR_HEADS; return c; }
  // total elements and the flat index of the last element must fit in 63 bits
  const long double elems = (long double)B * Hq * S * D;
  if (elems > 4.0e18L) { c.status = ATTN_ERR_SHAPE; return c; }
  if (mask_kind == ATTN_MASK_CAUSAL_WINDOW && window < 1) { c.status = ATTN_ERR_WINDOW; return c; }
  if (mask_kind == ATTN_MASK_LOCAL_GLOBAL && window < 0) { c.status = ATTN_ERR_WINDOW; return c; }
  if (n_global < 0 || n_global > ATTN_MAX_GLOBAL) { c.status = ATTN_ERR_GLOBAL; return c; }
  if (n_global > 0 && (mask_kind != ATTN_MASK_LOCAL_GLOBAL || global_idx == nullptr)) {
    c.status = ATTN_ERR_GLOBAL;
    return c;
  }
  int tmp[ATTN_MAX_GLOBAL];
  for (int i = 0; i < n_global; ++i) {
    if (global_idx[i] < 0 || global_idx[i] >= S) { c.status = ATTN_ERR_GLOBAL; return c; }
    tmp[i] = global_idx[i];
  }
  std::sort(tmp, tmp + n_global);
  const int nd = (int)(std::unique(tmp, tmp + n_global) - tmp);
  std::copy(tmp, tmp + nd, c.gpos);
  c.n_global = nd;

  if (dtype == ATTN_DTYPE_FP32)
    c.s = attn::make_sched(B, Hq, Hkv, S, mask_kind, window, nd, attn::kF32Rows, attn::kF32Keys, 0,
                           attn::kF32Rows);
  else  // (the FP8 kernel's tiles are 128 keys at either head width)
    c.s = attn::make_sched(B, Hq, Hkv, S, mask_kind, window, nd, attn::kBf16Rows,
                           fp8 ? 128 : attn::bf16_keys_per_tile(D), 1, attn::kBf16GlobalRows);
  if (c.s.n_items > 0x7fffffffLL) { c.status = ATTN_ERR_SHAPE; return c; }
  return c;
}

// Compute units of the device a stream launches on (cached per device; 0 when
// the runtime cannot tell, which keeps the one-workgroup-per-item launch).
// The device a stream belongs to (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  return stream ? hipStreamGetDevice(stream, dev) : hipGetDevice(dev);
}

int device_cus(hipStream_t stream) {
  static std::atomic<int> cache[64];
  int dev = -1;
  if (stream_device(stream, &dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Exact visible (query, key) pairs of one head, from per-row closed forms.
long long visible_pairs(int S, int mask, int window, const int* g, int ng) {
  const long long n = S;
  switch (mask) {
    case ATTN_MASK_FULL: return n * n;
    case ATTN_MASK_CAUSAL: return n * (n + 1) / 2;
    case ATTN_MASK_CAUSAL_WINDOW: {
      const long long w = std::min<long long>(window, n);
      return w * (w + 1) / 2 + (n - w) * w;  // rows i < w see i+1 keys, the rest w
    }
    default: {
      long long tot = 0;
      const long long w = window;
      for (long long i = 0; i < n; ++i) {
        bool is_g = std::binary_search(g, g + ng, (int)i);
        if (is_g) { tot += n; continue; }
        long long band = std::min(i, w) + std::min(n - 1 - i, w) + 1;
        for (int t = 0; t < ng; ++t) {
          long long d = i - g[t];
          if (d > w || -d > w) ++band;
        }
        tot += band;
      }
      return tot;
    }
  }
}

struct DecodePlan {
  int status;
  int window;        // the sliding window clamped to Smax, 0 without one
  int uni_splits;    // splits of every pair when all sequences hold Smax positions
  int grid_uniform;  // workgroups without lengths: pairs x uni_splits
  int grid_ragged;   // workgroups with device lengths: max(kDecodeWorkgroups, pairs),
                     // a bound on the items of the kernel's plan
  size_t hdr_off;    // bytes from the workspace start to the per-pair header
  size_t ws_bytes;
};

// Validation and the key-split plan of a decode call.  The key range of a
// sequence is its last min(L, w + Sq - 1) positions under a window of w, all
// L otherwise.  Splits hold at least kDecodeMinTiles tiles, and the work items
// (pairs x splits) of a plan fit in kDecodeWorkgroups whenever the pairs do.
// Without device lengths every pair holds the same tiles and the splits are
// planned here; with them the kernel plans from the lengths, and the grid and
// the workspace take the bounds of its plan: at most max(kDecodeWorkgroups,
// pairs) items, and at most kDecodeWorkgroups partial slots (only pairs with
// two or more splits take them).  Neither depends on the lengths, so they
// may change from call to call without a new workspace.
DecodePlan plan_decode(int B, int Hq, int Hkv, int Sq, int Smax, int D, int mask_kind,
                       int window, int dtype) {
  DecodePlan d{};
  d.status = ATTN_OK;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Smax < 1 || (long long)Smax > kMaxS) {
    d.status = ATTN_ERR_SHAPE;
    return d;
  }
  if (dtype != ATTN_DTYPE_BF16) { d.status = ATTN_ERR_UNSUPPORTED; return d; }
  if (D != 64 && D != 128) { d.status = ATTN_ERR_UNSUPPORTED; return d; }
  if (mask_kind != ATTN_MASK_FULL && mask_kind != ATTN_MASK_CAUSAL &&
      mask_kind != ATTN_MASK_CAUSAL_WINDOW) {
    d.status = ATTN_ERR_UNSUPPORTED;
    return d;
  }
  if (mask_kind == ATTN_MASK_CAUSAL_WINDOW ? window < 1 : window != 0) {
    d.status = ATTN_ERR_WINDOW;
    return d;
  }
  if (Hq % Hkv != 0) { d.status = ATTN_ERR_HEADS; return d; }
  if ((long long)(Hq / Hkv) * Sq > attn::kDecodeRows) { d.status = ATTN_ERR_UNSUPPORTED; return d; }
  const long double elems = (long double)B * std::max(Hq, Hkv) * std::max(Sq, Smax) * D;
  if (elems > 4.0e18L) { d.status = ATTN_ERR_SHAPE; return d; }
  d.window = std::min(window, Smax);  // a window of Smax or more sees every causal position
  const long long pairs = (long long)B * Hkv;
  const long long keys = d.window ? std::min<long long>(Smax, (long long)d.window + Sq - 1) : Smax;
  const int tiles = (int)((keys + attn::kDecodeTile - 1) / attn::kDecodeTile);
  d.uni_splits = (int)std::max<long long>(
      1, std::min<long long>(attn::cdiv(tiles, attn::kDecodeMinTiles), attn::kDecodeWorkgroups / pairs));
  const long long grid_u = pairs * d.uni_splits;
  const long long grid_r = std::max<long long>(attn::kDecodeWorkgroups, pairs);
  if (std::max(grid_u, grid_r) > 0x7fffffffLL || pairs * attn::kDecodeRows > 0x7fffffffLL) {
    d.status = ATTN_ERR_SHAPE;  // grid sizes of the two kernels
    return d;
  }
  d.grid_uniform = (int)grid_u;
  d.grid_ragged = (int)grid_r;
  if (tiles > attn::kDecodeMinTiles) {  // some pair may take two or more splits
    const size_t slot = (size_t)attn::kDecodeRows * (size_t)(D + 2) * sizeof(float);
    d.hdr_off = (size_t)attn::kDecodeWorkgroups * slot;
    d.ws_bytes = d.hdr_off + (size_t)pairs * 2 * sizeof(int);
  }
  return d;
}

}  // namespace

// Static device scratch behind attn_decode_noalloc: one copy per GPU.  In
// host code the array's name is only a stand-in; every use goes through the
// address hipGetSymbolAddress returned for the device (kept in g_scratch).
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of `scratch`, looked up on the first call with the
// device current (the caller's current device is restored).
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      int cur = -1;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess) return e;
      if (!ptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

// attn_decode (static_scratch false: the caller's workspace) and
// attn_decode_noalloc (true: this device's copy of `scratch`).
int decode_call(const void* q, const void* k_cache, const void* v_cache, void* o,
                const int* cache_len, int B, int Hq, int Hkv, int Sq, int Smax, int D,
                int mask_kind, int window, float scale, int dtype, void* workspace,
                size_t workspace_bytes, hipStream_t stream, bool static_scratch) {
  if (!q || !k_cache || !v_cache || !o) return ATTN_ERR_NULL;
  const DecodePlan d = plan_decode(B, Hq, Hkv, Sq, Smax, D, mask_kind, window, dtype);
  if (d.status != ATTN_OK) return d.status;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  for (const void* ptr : {q, k_cache, v_cache, (const void*)o})
    if ((uintptr_t)ptr % 16 != 0) return ATTN_ERR_ALIGN;
  if (cache_len && (uintptr_t)cache_len % 4 != 0) return ATTN_ERR_ALIGN;
  const size_t nq = (size_t)B * Hq * Sq * D * 2, nkv = (size_t)B * Hkv * Smax * D * 2;
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k_cache, nkv) || overlaps(o, nq, v_cache, nkv))
    return ATTN_ERR_ALIAS;
  if (static_scratch && d.ws_bytes > 0) {
    if (d.ws_bytes > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    int dev = -1;
    if (stream_device(stream, &dev) != hipSuccess) return ATTN_ERR_HIP;
    if (scratch_address(dev, &workspace) != hipSuccess) return ATTN_ERR_HIP;
    workspace_bytes = ATTN_NOALLOC_SCRATCH_BYTES;
  }
  const bool split = cache_len ? d.ws_bytes > 0 : d.uni_splits > 1;
  if (d.ws_bytes > 0) {
    if (!workspace || workspace_bytes < d.ws_bytes || (uintptr_t)workspace % 16 != 0)
      return ATTN_ERR_WORKSPACE;
    if (overlaps(workspace, d.ws_bytes, o, nq) || overlaps(workspace, d.ws_bytes, q, nq) ||
        overlaps(workspace, d.ws_bytes, k_cache, nkv) || overlaps(workspace, d.ws_bytes, v_cache, nkv))
      return ATTN_ERR_ALIAS;
  }

  attn::DParams p{};
  p.q = q; p.k = k_cache; p.v = v_cache; p.o = o;
  p.cache_len = cache_len;
  p.ws = split ? (float*)workspace : nullptr;
  p.hdr = split ? (int*)((char*)workspace + d.hdr_off) : nullptr;
  p.max_slots = split ? attn::kDecodeWorkgroups : 0;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Smax = Smax; p.G = Hq / Hkv;
  p.uni_splits = cache_len ? 0 : d.uni_splits;
  p.causal = mask_kind != ATTN_MASK_FULL ? 1 : 0;
  p.window = d.window;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  p.qmode = scale > 0.f ? 0 : (scale < 0.f ? 1 : 2);
  if (p.qmode == 2) p.c = 1.f;  // all visible scores equal: weights are uniform
  hipError_t err = attn::launch_decode(p, D, cache_len ? d.grid_ragged : d.grid_uniform, stream);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int S,
             int D, int mask_kind, int window, const int* global_idx, int n_global, float scale,
             int dtype, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  Checked c = check_args(B, Hq, Hkv, S, D, mask_kind, window, global_idx, n_global, dtype);
  if (c.status != ATTN_OK) return c.status;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  for (const void* ptr : {q, k, v, (const void*)o})
    if ((uintptr_t)ptr % 16 != 0) return ATTN_ERR_ALIGN;
  // element sizes of the inputs and of the output (FP8 writes bf16)
  const size_t esz = dtype == ATTN_DTYPE_FP32 ? 4 : dtype == ATTN_DTYPE_BF16 ? 2 : 1;
  const size_t osz = dtype == ATTN_DTYPE_FP32 ? 4 : 2;
  const size_t nq = (size_t)B * Hq * S * D * esz, nkv = (size_t)B * Hkv * S * D * esz;
  const size_t no = (size_t)B * Hq * S * D * osz;
  if (overlaps(o, no, q, nq) || overlaps(o, no, k, nkv) || overlaps(o, no, v, nkv))
    return ATTN_ERR_ALIAS;

  KParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o;
  p.s = c.s;
  p.scale = scale;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  p.qmode = scale > 0.f ? 0 : (scale < 0.f ? 1 : 2);
  if (p.qmode == 2) p.c = 1.f;  // all visible scores equal: weights are uniform
  std::copy(c.gpos, c.gpos + c.n_global, p.gpos);

  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  if (dtype == ATTN_DTYPE_BF16 && D == 128 && mask_kind != ATTN_MASK_LOCAL_GLOBAL &&
      p.qmode == 0) {
    // more items than CUs: one persistent workgroup per CU walks them (the
    // persistent kernel takes q as given, so negative and zero scales, which
    // flip or zero q, keep the one-workgroup-per-item launch)
    const int cus = device_cus(st);
    err = (cus > 0 && c.s.n_items > cus) ? attn::launch_bf16_pers_d128(p, cus, st)
                                         : attn::launch_bf16_d128(p, st);
  } else {
    err = dtype == ATTN_DTYPE_BF16
              ? (D == 64 ? attn::launch_bf16_d64(p, st) : attn::launch_bf16_d128(p, st))
          : dtype != ATTN_DTYPE_FP32 ? attn::launch_fp8(p, D, dtype == ATTN_DTYPE_FP8_E5M2, st)
                                         : attn::launch_fp32(p, D, st);
  }
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_ex(const attn_fwd_args* a, void* stream) {
  if (!a) return ATTN_ERR_NULL;
  if (!a->q || !a->k || !a->v || !a->o) return ATTN_ERR_NULL;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Sq < 1 || a->Skv < 1 || (long long)a->Sq > kMaxS ||
      (long long)a->Skv > kMaxS)
    return ATTN_ERR_SHAPE;
  if (a->dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED;
  if (a->D != 64 && a->D != 128) return ATTN_ERR_UNSUPPORTED;
  if (a->mask_kind < ATTN_MASK_FULL || a->mask_kind > ATTN_MASK_LOCAL_GLOBAL)
    return ATTN_ERR_UNSUPPORTED;
  // local+global: not with ALiBi, a block-sparse layout or a distance bias;
  // a distance bias: not with ALiBi or a layout either
  if (a->mask_kind == ATTN_MASK_LOCAL_GLOBAL &&
      (a->alibi_slopes || a->block_layout || a->dist_bias))
    return ATTN_ERR_UNSUPPORTED;
  if (a->dist_bias && (a->alibi_slopes || a->block_layout)) return ATTN_ERR_UNSUPPORTED;
  // distance-bias rows of Sq + Skv - 1 fp32 values, byte offsets in 31 bits
  if (a->dist_bias && (long long)a->Sq + a->Skv > (1LL << 29)) return ATTN_ERR_SHAPE;
  if (a->Hq % a->Hkv != 0) return ATTN_ERR_HEADS;
  if (a->mask_kind == ATTN_MASK_CAUSAL_WINDOW && a->window < 1) return ATTN_ERR_WINDOW;
  if (a->mask_kind == ATTN_MASK_LOCAL_GLOBAL && a->window < 0) return ATTN_ERR_WINDOW;
  // local+global: positions -Sq .. Skv - 1 and windows up to Sq + Skv in 32 bits
  if (a->mask_kind == ATTN_MASK_LOCAL_GLOBAL && (long long)a->Sq + a->Skv >= (1LL << 30))
    return ATTN_ERR_SHAPE;
  // global key positions: local+global only, in [0, Skv), sorted and made distinct
  if (a->n_global < 0 || a->n_global > ATTN_MAX_GLOBAL) return ATTN_ERR_GLOBAL;
  if (a->n_global > 0 && (a->mask_kind != ATTN_MASK_LOCAL_GLOBAL || a->global_idx == nullptr))
    return ATTN_ERR_GLOBAL;
  int gpos[ATTN_MAX_GLOBAL];
  for (int i = 0; i < a->n_global; ++i) {
    if (a->global_idx[i] < 0 || a->global_idx[i] >= a->Skv) return ATTN_ERR_GLOBAL;
    gpos[i] = a->global_idx[i];
  }
  std::sort(gpos, gpos + a->n_global);
  const int n_global = (int)(std::unique(gpos, gpos + a->n_global) - gpos);
  if (!std::isfinite(a->scale)) return ATTN_ERR_SCALE;
  for (const void* ptr : {a->q, a->k, a->v, (const void*)a->o})
    if ((uintptr_t)ptr % 16 != 0) return ATTN_ERR_ALIGN;
  for (const void* ptr : {(const void*)a->alibi_slopes, (const void*)a->q_len,
                          (const void*)a->kv_len, (const void*)a->block_layout,
                          (const void*)a->dist_bias})
    if ((uintptr_t)ptr % 4 != 0) return ATTN_ERR_ALIGN;
  // block-sparse layouts: square, at most ATTN_SPARSE_MAX_BLOCKS blocks, full or
  // causal mask, no bias or lengths
  if (a->block_layout &&
      (a->Sq != a->Skv || a->Sq > ATTN_SPARSE_MAX_BLOCKS * ATTN_SPARSE_BLOCK ||
       a->mask_kind == ATTN_MASK_CAUSAL_WINDOW || a->alibi_slopes || a->q_len || a->kv_len))
    return ATTN_ERR_UNSUPPORTED;
  // ALiBi slopes and distance biases are turned into score units by 1 / |scale|
  if ((a->alibi_slopes || a->dist_bias) && a->scale != 0.f && std::fabs(a->scale) < 0x1p-60f)
    return ATTN_ERR_SCALE;
  const long long* strides[4] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
  for (const long long* st : strides) {
    for (int d = 0; d < 3; ++d)
      if (st[d] < 0 || st[d] % 8 != 0) return ATTN_ERR_ALIGN;
    if (st[2] > (1LL << 23)) return ATTN_ERR_SHAPE;
  }
  // byte extents [ptr, ptr + span) of the four tensors
  auto span = [&](const long long* st, int H, int S) {
    return (size_t)(((long double)(a->B - 1) * st[0] + (long double)(H - 1) * st[1] +
                     (long double)(S - 1) * st[2] + a->D) * 2);
  };
  const long double big = (long double)(a->B) * std::max(a->Hq, a->Hkv) *
                          std::max(a->Sq, a->Skv) * a->D;
  if (big > 4.0e18L) return ATTN_ERR_SHAPE;
  const size_t nq = span(a->q_stride, a->Hq, a->Sq), nk = span(a->k_stride, a->Hkv, a->Skv);
  const size_t nv = span(a->v_stride, a->Hkv, a->Skv), no = span(a->o_stride, a->Hq, a->Sq);
  if (overlaps(a->o, no, a->q, nq) || overlaps(a->o, no, a->k, nk) || overlaps(a->o, no, a->v, nv))
    return ATTN_ERR_ALIAS;
  if ((a->alibi_slopes && overlaps(a->o, no, a->alibi_slopes, (size_t)a->Hq * 4)) ||
      (a->q_len && overlaps(a->o, no, a->q_len, (size_t)a->B * 4)) ||
      (a->kv_len && overlaps(a->o, no, a->kv_len, (size_t)a->B * 4)) ||
      (a->dist_bias &&
       overlaps(a->o, no, a->dist_bias, (size_t)a->Hq * ((size_t)a->Sq + a->Skv - 1) * 4)))
    return ATTN_ERR_ALIAS;
  const int lay_nb = (a->Sq + ATTN_SPARSE_BLOCK - 1) / ATTN_SPARSE_BLOCK;
  const int lay_nw = ATTN_LAYOUT_WORDS(lay_nb);
  if (a->block_layout && overlaps(a->o, no, a->block_layout, (size_t)lay_nb * lay_nw * 4))
    return ATTN_ERR_ALIAS;
  // o's own rows must be distinct: rows of one head D apart at least, heads and
  // batches not folded onto each other
  const long long* os = a->o_stride;
  if (os[2] < a->D || (a->Hq > 1 && os[1] < (long long)a->Sq * os[2] && os[2] < (long long)a->Hq * os[1]) ||
      (a->B > 1 && os[0] == 0) || (a->Hq > 1 && os[1] == 0))
    return ATTN_ERR_ALIAS;

  // A window of Skv keys or more admits every key at or before the query (a
  // query's key position is at most Skv - 1), so larger causal windows are
  // clamped to Skv; a band of radius Sq + Skv holds every key of every query
  // (positions run from -Sq to Skv - 1), so larger local+global windows are
  // clamped to that (such calls have Sq + Skv below 2^30).  The kernels then
  // form position +- window in 32-bit arithmetic without overflow.
  const int window = a->mask_kind == ATTN_MASK_CAUSAL_WINDOW ? std::min(a->window, a->Skv)
                     : a->mask_kind == ATTN_MASK_LOCAL_GLOBAL ? std::min(a->window, a->Sq + a->Skv)
                                                              : 0;
  Sched s = attn::make_sched(a->B, a->Hq, a->Hkv, a->Sq, a->mask_kind, window, n_global,
                             attn::kBf16Rows, attn::bf16_keys_per_tile(a->D), 1,
                             attn::kBf16GlobalRows);
  if (s.n_items > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  s.Sk = a->Skv;
  s.off = a->Skv - a->Sq;

  KParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o;
  p.s = s;
  p.scale = a->scale;
  p.c = std::fabs(a->scale) * 1.4426950408889634f;
  p.qmode = a->scale > 0.f ? 0 : (a->scale < 0.f ? 1 : 2);
  if (p.qmode == 2) p.c = 1.f;
  p.general = 1;
  p.qlen = a->q_len;
  p.kvlen = a->kv_len;
  p.slopes = a->alibi_slopes;
  p.bias_k = a->scale != 0.f ? 1.f / std::fabs(a->scale) : 1.4426950408889634f;
  p.bias = a->dist_bias;
  p.bias_len = a->Sq + a->Skv - 1;
  p.layout = a->block_layout;
  p.lay_nw = lay_nw;
  std::copy(gpos, gpos + n_global, p.gpos);
  for (int d = 0; d < 3; ++d) {
    p.qs[d] = a->q_stride[d];
    p.ks[d] = a->k_stride[d];
    p.vs[d] = a->v_stride[d];
    p.os[d] = a->o_stride[d];
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t err = a->D == 64 ? attn::launch_bf16_d64(p, st) : attn::launch_bf16_d128(p, st);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_plan(int B, int Hq, int Hkv, int S, int D, int mask_kind, int window,
              const int* global_idx, int n_global, int dtype, attn_plan_info* info) {
  if (!info) return ATTN_ERR_NULL;
  Checked c = check_args(B, Hq, Hkv, S, D, mask_kind, window, global_idx, n_global, dtype);
  if (c.status != ATTN_OK) return c.status;
  const Sched& s = c.s;
  attn_plan_info r{};
  r.work_items = s.n_items;
  r.rows_per_item = s.BMh;
  r.heads_per_item = s.HP;
  r.keys_per_tile = s.BN;
  r.kernel = dtype == ATTN_DTYPE_BF16 ? 1 : dtype == ATTN_DTYPE_FP32 ? 0 : 2;
  // Walk one pair's items (all pairs are alike) and scale by the pair count.
  long long visits = 0, partial = 0;
  for (long long id = 0; id < s.n_items; id += s.P) {
    attn::Item it = attn::decode_item(s, (int)id);
    int r0 = 0, r1 = 0;
    if (!it.is_global) { r0 = it.blk * s.BMh; r1 = std::min(r0 + s.BMh, s.S) - 1; }
    int klo, khi;
    attn::key_range(s, it.is_global, r0, r1, &klo, &khi);
    const int kt_lo = klo / s.BN, kt_hi = khi / s.BN;
    const int strip = (!it.is_global && s.n_global > 0) ? attn::cdiv(s.n_global, s.BN) : 0;
    visits += (kt_hi - kt_lo + 1) + strip;
    partial += strip;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      int cls = it.is_global ? ((long long)kt * s.BN + s.BN > s.S ? attn::TILE_PARTIAL : attn::TILE_FULL)
                             : attn::classify_tile(s.mask, s.window, s.S, r0, r1, kt * s.BN, s.BN);
      if (cls == attn::TILE_PARTIAL) ++partial;
    }
  }
  r.tile_visits = visits * s.P;
  r.partial_tiles = partial * s.P;
  r.visible_pairs = visible_pairs(S, mask_kind, window, c.gpos, c.n_global);
  r.effective_flops = 4.0 * D * (double)r.visible_pairs * B * Hq;
  *info = r;
  return ATTN_OK;
}

int attn_decode_workspace(int B, int Hq, int Hkv, int Sq, int Smax, int D, int mask_kind,
                          int window, int dtype, size_t* workspace_bytes) {
  if (!workspace_bytes) return ATTN_ERR_NULL;
  const DecodePlan d = plan_decode(B, Hq, Hkv, Sq, Smax, D, mask_kind, window, dtype);
  if (d.status != ATTN_OK) return d.status;
  *workspace_bytes = d.ws_bytes;
  return ATTN_OK;
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                const int* cache_len, int B, int Hq, int Hkv, int Sq, int Smax, int D,
                int mask_kind, int window, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return decode_call(q, k_cache, v_cache, o, cache_len, B, Hq, Hkv, Sq, Smax, D, mask_kind, window,
                     scale, dtype, workspace, workspace_bytes, (hipStream_t)stream, false);
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                        const int* cache_len, int B, int Hq, int Hkv, int Sq, int Smax, int D,
                        int mask_kind, int window, float scale, int dtype, void* stream) {
  return decode_call(q, k_cache, v_cache, o, cache_len, B, Hq, Hkv, Sq, Smax, D, mask_kind, window,
                     scale, dtype, nullptr, 0, (hipStream_t)stream, true);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_HEADS: return "ATTN_ERR_HEADS";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WINDOW: return "ATTN_ERR_WINDOW";
    case ATTN_ERR_GLOBAL: return "ATTN_ERR_GLOBAL";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS";
    case ATTN_ERR_SCALE: return "ATTN_ERR_SCALE";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_SCRATCH: return "ATTN_ERR_SCRATCH";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

int attn_version(void) { return kVersion; }

}  // extern "C"
