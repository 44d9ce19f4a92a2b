// gfx950_ops.h -- small device helpers shared by the bf16 attention kernels:
// vector types, the 32x32x16 bf16 MFMA, v_max3 and lane-pair max, LDS-direct
// (global/buffer -> LDS) loads, and LDS operand reads issued as inline asm with
// explicit lgkmcnt waits.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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

// Wait until at most N LDS reads are outstanding, tied to the operand f so
// that no use of it is scheduled above the wait.
template <int N>
__device__ __forceinline__ void lds_wait1(bf16x8& f) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f) : "i"(N));
}

}  // namespace
}  // namespace attn
