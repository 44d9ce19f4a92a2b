// attn_layout.cpp -- host builders of block-sparse layouts for attn_fwd_ex.
//
// A layout is a bitmask over blocks of ATTN_SPARSE_BLOCK positions: row I
// (query block) holds ATTN_LAYOUT_WORDS(nb) 32-bit words, bit J % 32 of word
// J / 32 set when query block I may look at key block J.  The patterns are
// those of "第 8 章 AI 算法Transformer大模型", section 8.3 (8.3.1 strided and
// fixed, 8.3.3 Big Bird), applied to blocks as the block-sparse kernels of
// section 8.3.4 do:
//   strided  J <= I, and I - J <= local or I - J a multiple of stride
//   fixed    J <= I, and J in I's chunk of `chunk` blocks, or J % chunk == I % chunk
//   bigbird  |I - J| <= radius, or J < n_global, or I < n_global, or J in rand[I]
#include <cstdint>
#include <cstring>

#include "../../include/attn.h"

namespace {

inline void set_bit(uint32_t* row, int j) { row[j >> 5] |= 1u << (j & 31); }

bool valid_nb(int nb) { return nb >= 1 && nb <= ATTN_SPARSE_MAX_BLOCKS; }

}  // namespace

extern "C" {

int attn_layout_strided(int nb, int local_blocks, int stride_blocks, uint32_t* layout) {
  if (!layout) return ATTN_ERR_NULL;
  if (!valid_nb(nb) || local_blocks < 0 || stride_blocks < 1) return ATTN_ERR_SHAPE;
  const int nw = ATTN_LAYOUT_WORDS(nb);
  std::memset(layout, 0, sizeof(uint32_t) * (size_t)nb * nw);
  for (int I = 0; I < nb; ++I)
    for (int J = 0; J <= I; ++J)
      if (I - J <= local_blocks || (I - J) % stride_blocks == 0) set_bit(layout + (size_t)I * nw, J);
  return ATTN_OK;
}

int attn_layout_fixed(int nb, int chunk_blocks, uint32_t* layout) {
  if (!layout) return ATTN_ERR_NULL;
  if (!valid_nb(nb) || chunk_blocks < 1) return ATTN_ERR_SHAPE;
  const int nw = ATTN_LAYOUT_WORDS(nb);
  std::memset(layout, 0, sizeof(uint32_t) * (size_t)nb * nw);
  for (int I = 0; I < nb; ++I)
    for (int J = 0; J <= I; ++J)
      if (J / chunk_blocks == I / chunk_blocks || J % chunk_blocks == I % chunk_blocks)
        set_bit(layout + (size_t)I * nw, J);
  return ATTN_OK;
}

int attn_layout_bigbird(int nb, int radius_blocks, int n_global_blocks, const int* rand_blocks,
                        int n_rand, uint32_t* layout) {
  if (!layout || (n_rand > 0 && !rand_blocks)) return ATTN_ERR_NULL;
  if (!valid_nb(nb) || radius_blocks < 0 || n_global_blocks < 0 || n_rand < 0)
    return ATTN_ERR_SHAPE;
  for (long long t = 0; t < (long long)nb * n_rand; ++t)
    if (rand_blocks[t] < 0 || rand_blocks[t] >= nb) return ATTN_ERR_SHAPE;
  const int nw = ATTN_LAYOUT_WORDS(nb);
  std::memset(layout, 0, sizeof(uint32_t) * (size_t)nb * nw);
  for (int I = 0; I < nb; ++I) {
    uint32_t* row = layout + (size_t)I * nw;
    for (int J = 0; J < nb; ++J) {
      const int d = I > J ? I - J : J - I;
      if (d <= radius_blocks || J < n_global_blocks || I < n_global_blocks) set_bit(row, J);
    }
    for (int t = 0; t < n_rand; ++t) set_bit(row, rand_blocks[(size_t)I * n_rand + t]);
  }
  return ATTN_OK;
}

}  // extern "C"
