/*
 * attn.h -- C ABI of libattn.so: fused masked / grouped-query scaled
 * dot-product attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * Operation ("Trasformer 浅析", section 缩放点积注意力; shapes and head map from
 * "Transformer 架构及其变体", section 带显式形状的因果自注意力):
 *
 *   for every batch b, query head a, query position i:
 *     h      = a / (Hq / Hkv)                       key/value head of query head a
 *     s_ij   = scale * sum_d q[b][a][i][d] * k[b][h][j][d]      for visible j
 *     p_ij   = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
 *     o[b][a][i][:] = sum_j p_ij * v[b][h][j][:]
 *
 * Masked pairs are excluded exactly (their weight is zero), as with the -inf
 * mask entries of "Trasformer 浅析", section 掩码与三种架构范式.
 *
 * Layout: q and o are [B][Hq][S][D], k and v are [B][Hkv][S][D], dense
 * row-major (D fastest), all four in the same element type, all in device
 * memory owned by the caller.  The n x n score matrix is never stored: the
 * library allocates no device memory at all.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Which (query i, key j) pairs are visible. */
typedef enum {
  ATTN_MASK_FULL = 0,          /* every key (bidirectional)                        */
  ATTN_MASK_CAUSAL = 1,        /* j <= i  ("Trasformer 浅析", causal-mask equation) */
  ATTN_MASK_CAUSAL_WINDOW = 2, /* i - window < j <= i: the last `window` keys up to
                                  and including i; window >= 1                     */
  ATTN_MASK_LOCAL_GLOBAL = 3   /* |i - j| <= window, or i is a global token, or j is
                                  a global token ("Transformer 演进与变体", section
                                  稀疏注意力, sliding window of radius w plus global
                                  tokens); window >= 0                            */
} attn_mask_kind;

/* Element type of q, k, v and o.  Arithmetic: bf16 products accumulate in fp32
 * on the matrix cores; softmax statistics are fp32; the attention weights are
 * rounded to bf16 (nearest even) before the P.V product; o is rounded once to
 * bf16 at the end.  fp32 inputs are computed entirely in fp32. */
typedef enum {
  ATTN_DTYPE_FP32 = 0,
  ATTN_DTYPE_BF16 = 1,
  /* q, k, v as OCP E4M3 bytes, o as bf16: attn_fwd only, D = 64 or 128, every
   * mask ("Transformer 演进与变体", section Flash
   * Attention, the FlashAttention-3 paragraph: FP8 operands for both matrix
   * products, softmax and accumulation in higher precision).  Both products
   * run on the FP8 matrix cores (the instruction truncates the smaller
   * products of each group of 8 to 13 bits below the group's largest, then
   * accumulates in fp32); P is rounded to E4M3 (nearest even) for the second.  Per-tensor scale factors stay with the
   * caller: fold q's and k's into `scale`, multiply o by v's. */
  ATTN_DTYPE_FP8_E4M3 = 2,
  /* the same with q, k, v as OCP E5M2 bytes (the other FP8 format that
   * paragraph names: two mantissa bits, five exponent bits, infinities); the
   * weights P stay E4M3 for the P.V product (they lie in [0, 2^8), where
   * E4M3's extra mantissa bit counts and E5M2's range does not) */
  ATTN_DTYPE_FP8_E5M2 = 3
} attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                          */
  ATTN_ERR_SHAPE = 2,       /* B, Hq, Hkv or S < 1, or sizes overflow              */
  ATTN_ERR_HEADS = 3,       /* Hq is not a multiple of Hkv                         */
  ATTN_ERR_UNSUPPORTED = 4, /* D not in {64, 128}, unknown dtype or mask kind      */
  ATTN_ERR_WINDOW = 5,      /* window out of range for the mask kind               */
  ATTN_ERR_GLOBAL = 6,      /* bad global tokens: n_global out of [0, 64], index out
                               of [0, S), or globals given with another mask kind  */
  ATTN_ERR_ALIGN = 7,       /* a tensor pointer is not 16-byte aligned             */
  ATTN_ERR_HIP = 8,         /* the kernel launch failed (hipGetLastError)          */
  ATTN_ERR_ALIAS = 9,       /* o overlaps q, k or v                                */
  ATTN_ERR_SCALE = 10,      /* scale is NaN or infinite                            */
  ATTN_ERR_WORKSPACE = 11,  /* attn_decode: workspace missing, smaller than
                               attn_decode_workspace reports, or not 16-byte aligned */
  ATTN_ERR_SCRATCH = 12     /* attn_decode_noalloc: the call needs more than the
                               library's static device scratch (ATTN_NOALLOC_SCRATCH_BYTES) */
} attn_status;

#define ATTN_MAX_GLOBAL 64

/* Block-sparse layouts (attn_fwd_ex's block_layout): blocks of 64 positions,
 * at most 512 blocks (32768 positions); row I of a layout holds
 * ATTN_LAYOUT_WORDS(nb) uint32 words, bit J % 32 of word J / 32 set when query
 * block I may look at key block J. */
#define ATTN_SPARSE_BLOCK 64
#define ATTN_SPARSE_MAX_BLOCKS 512
#define ATTN_LAYOUT_WORDS(nb) (((nb) + 31) / 32)

/*
 * attn_fwd -- enqueue the attention forward pass on `stream`.
 *
 *   q, k, v     device pointers, layouts above, read only
 *   o           device pointer [B][Hq][S][D], written; must not overlap q, k, v
 *   B, Hq, Hkv  batch, query heads, key/value heads (Hq % Hkv == 0;
 *               Hkv == Hq is multi-head, Hkv == 1 is multi-query attention)
 *   S           sequence length (any S >= 1; partial tiles are handled)
 *   D           head width, 64 or 128
 *   mask_kind   attn_mask_kind
 *   window      ignored for FULL and CAUSAL; see attn_mask_kind otherwise
 *   global_idx  HOST pointer to n_global int32 positions (LOCAL_GLOBAL only);
 *               treated as a set (order and duplicates do not matter), read
 *               during the call and not kept; may be NULL when n_global == 0
 *   n_global    number of entries in global_idx, 0..ATTN_MAX_GLOBAL
 *   scale       multiplies q.k; used exactly as given (0 gives uniform weights;
 *               the usual choice is 1/sqrt(D), "Trasformer 浅析", section
 *               缩放因子的必要性)
 *   dtype       attn_dtype of all four tensors (ATTN_DTYPE_FP8_E4M3 and _E5M2:
 *               q, k, v one byte per element, o bf16)
 *   stream      hipStream_t to launch on (NULL = the default stream)
 *
 * Returns ATTN_OK after enqueuing one kernel; the call does not synchronise.
 * Argument errors are detected on the host before any launch and leave o
 * untouched.  Faults during execution surface at the caller's next
 * synchronisation.  NaN/Inf inputs propagate.  Stateless and re-entrant; for a
 * given input the output is bitwise reproducible (no atomics in the numerics).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o,
             int B, int Hq, int Hkv, int S, int D,
             int mask_kind, int window, const int* global_idx, int n_global,
             float scale, int dtype, void* stream);

/*
 * attn_fwd_ex -- the forward pass with separate query and key lengths and
 * strided layouts (bf16).
 *
 * Queries q[b][a][i] (i < Sq) attend to keys and values k, v[b][h][j]
 * (j < Skv), h = a / (Hq / Hkv).  Cross attention ("Trasformer 浅析", section
 * 交叉注意力: queries from one sequence, keys and values from another) is
 * mask_kind FULL; a chunk of queries against a longer prefix ("Transformer
 * 架构及其变体", section 预填充创建缓存，解码复用缓存: a long prefill may run in
 * chunks) is CAUSAL or CAUSAL_WINDOW with the queries aligned to the END of
 * the keys: query i sits at key position p_i = i + Skv - Sq and sees
 *   CAUSAL          keys j <= p_i
 *   CAUSAL_WINDOW   keys p_i - window < j <= p_i
 *   FULL            every key
 *   LOCAL_GLOBAL    keys |p_i - j| <= window, every key when p_i is a global
 *                   position, and the global positions themselves (global_idx
 *                   holds key positions, the same for every sequence;
 *                   "Transformer 演进与变体", section 稀疏注意力, Longformer)
 * A query that sees no key (p_i < 0, possible when Skv < Sq) is written as
 * zeros.  With Sq == Skv and dense strides this is attn_fwd.
 *
 * Layouts: element (b, h, s, d) of each tensor is at
 *   ptr + b * stride[0] + h * stride[1] + s * stride[2] + d
 * (in elements; d contiguous).  [B][H][S][D] dense has strides
 * {H*S*D, S*D, D}; [B][S][H][D] (sequence-major) has {S*H*D, D, H*D}.
 * Strides must be non-negative multiples of 8 elements (16-byte rows), row
 * strides at most 2^23 elements; o's rows must not overlap each other or the
 * inputs.  fp32 returns ATTN_ERR_UNSUPPORTED here.
 *
 * Optional parts (NULL pointers leave them out):
 *   alibi_slopes  device, Hq fp32 slopes m_a: query head a adds -m_a * |p_i - j|
 *                 to each scaled score ("Transformer 演进与变体", section
 *                 线性偏置注意力; "Trasformer 浅析", section 加性偏置：ALiBi;
 *                 "Transformer 架构及其变体", section 位置信息通过查询和键进入注意力:
 *                 a per-head penalty linear in the query-key distance, added
 *                 after the 1/sqrt(d) scaling).  Slopes are read by the kernel;
 *                 any finite value works while m_a / |scale| stays far below
 *                 the fp32 range; a scale of magnitude below 2^-60 other than 0
 *                 returns ATTN_ERR_SCALE.
 *   q_len, kv_len device, B int32 each: sequence b holds q_len[b] valid query
 *                 rows and kv_len[b] valid keys at the start of its rows (a
 *                 right-padded batch, "Trasformer 浅析", section 填充掩码与因果
 *                 掩码: padded positions are masked out).  It is computed as
 *                 the call with Sq = q_len[b], Skv = kv_len[b] (so query i sits
 *                 at key position i + kv_len[b] - q_len[b]); padded keys are
 *                 never read into the result; padded query rows (i >= q_len[b])
 *                 are written as zeros.  Values are clamped to [0, Sq] and
 *                 [0, Skv]; read by the kernel, so a captured launch can be
 *                 replayed with new lengths.
 *   block_layout  device, nb x ATTN_LAYOUT_WORDS(nb) uint32, nb = ceil(Sq / 64):
 *                 block-sparse attention ("第 8 章 AI 算法Transformer大模型",
 *                 section 8.3: sparse patterns, run as block-sparse products
 *                 per 8.3.4).  Key j is visible from query i only when bit
 *                 j / 64 of row i / 64 is set, in addition to the mask kind.
 *                 Needs Sq == Skv <= 32768, mask FULL or CAUSAL, no ALiBi and
 *                 no lengths (else ATTN_ERR_UNSUPPORTED).  The attn_layout_*
 *                 builders below write the pages' patterns; any layout works.
 *                 A query whose row sees no key is written as zeros.
 *   dist_bias     device, Hq x (Sq + Skv - 1) fp32, row a contiguous: a bias
 *                 that is a function of the signed distance d = j - p_i (key
 *                 position minus query position), one per query head.  Entry
 *                 d + Skv - 1 of row a is added to query head a's scaled
 *                 score of every pair at distance d, before the softmax (the
 *                 unified view of "Trasformer 浅析", closing section: every
 *                 positional prior is a term b_ij added to the scaled logits;
 *                 here b_ij depends on the distance only).  In padded batches
 *                 the distances are those of each sequence's own positions,
 *                 so the same table serves every sequence.  ALiBi is the table
 *                 -m_a |d|; a bucketed or clipped relative bias is written out
 *                 per distance.  Masks FULL, CAUSAL and CAUSAL_WINDOW, not with
 *                 ALiBi or a layout (else ATTN_ERR_UNSUPPORTED); Sq + Skv at
 *                 most 2^29 (else ATTN_ERR_SHAPE); the same scale limit as
 *                 ALiBi.  Values are read by the kernel, entries of masked
 *                 pairs never reach the result, and NaN/Inf entries of
 *                 visible pairs propagate.
 */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, Hq, Hkv;
  int Sq;                 /* query rows per (batch, head)                 */
  int Skv;                /* key / value rows per (batch, head)           */
  int D;                  /* 64 or 128                                    */
  long long q_stride[3];  /* element strides of q's batch, head, row dims */
  long long k_stride[3];
  long long v_stride[3];
  long long o_stride[3];
  int mask_kind;          /* ATTN_MASK_FULL, _CAUSAL, _CAUSAL_WINDOW or
                             _LOCAL_GLOBAL (not with ALiBi or a layout)    */
  int window;             /* CAUSAL_WINDOW: >= 1; LOCAL_GLOBAL: >= 0       */
  float scale;
  int dtype;              /* ATTN_DTYPE_BF16                              */
  const float* alibi_slopes;  /* device [Hq] fp32, or NULL                */
  const int* q_len;           /* device [B] int32, or NULL (all Sq valid)  */
  const int* kv_len;          /* device [B] int32, or NULL (all Skv valid) */
  const uint32_t* block_layout; /* device block-sparse layout, or NULL       */
  const int* global_idx;  /* LOCAL_GLOBAL: host array of n_global global key
                             positions in [0, Skv) (duplicates allowed), or
                             NULL when n_global is 0                        */
  int n_global;           /* 0..ATTN_MAX_GLOBAL                            */
  const float* dist_bias; /* device [Hq][Sq + Skv - 1] fp32, or NULL      */
} attn_fwd_args;

/* Enqueue attn_fwd_ex on `stream`; same return and error conventions as
 * attn_fwd (no allocation, no synchronisation, errors before any launch). */
int attn_fwd_ex(const attn_fwd_args* args, void* stream);

/*
 * Block-sparse layout builders (host memory, no device access): write the
 * nb x ATTN_LAYOUT_WORDS(nb) words of a pattern of "第 8 章 AI 算法Transformer
 * 大模型", section 8.3, over blocks of ATTN_SPARSE_BLOCK positions.  Return
 * ATTN_ERR_NULL for a NULL output and ATTN_ERR_SHAPE for nb outside
 * [1, ATTN_SPARSE_MAX_BLOCKS] or a parameter out of range; `layout` is
 * caller-owned.
 *
 * attn_layout_strided  (8.3.1 strided: a local window plus every stride-th
 *                      position) query block I sees J <= I with I - J <=
 *                      local_blocks or I - J a multiple of stride_blocks (>= 1).
 * attn_layout_fixed    (8.3.1 fixed: the own block plus the same column of the
 *                      earlier blocks; the page's block is a chunk of
 *                      chunk_blocks layout blocks, its column a block's place
 *                      in the chunk) J <= I with J / chunk == I / chunk or
 *                      J % chunk == I % chunk.
 * attn_layout_bigbird  (8.3.3 Big Bird: window, random and global) |I - J| <=
 *                      radius_blocks, or J < n_global_blocks, or I <
 *                      n_global_blocks, or J one of the n_rand entries of row I
 *                      of rand_blocks (nb x n_rand host ints in [0, nb): the
 *                      random draw is the caller's).
 */
int attn_layout_strided(int nb, int local_blocks, int stride_blocks, uint32_t* layout);
int attn_layout_fixed(int nb, int chunk_blocks, uint32_t* layout);
int attn_layout_bigbird(int nb, int radius_blocks, int n_global_blocks, const int* rand_blocks,
                        int n_rand, uint32_t* layout);

/* Host-only description of the work attn_fwd would launch for these arguments
 * (the same validation as attn_fwd, no device access).  Counts are per call. */
typedef struct {
  long long work_items;      /* workgroups launched                                */
  long long tile_visits;     /* (work item, key tile) pairs processed               */
  long long partial_tiles;   /* tile visits that need the per-element mask          */
  long long visible_pairs;   /* exact visible (query, key) pairs of one query head  */
  double effective_flops;    /* 4 * D * visible_pairs * B * Hq                       */
  int rows_per_item;         /* query rows per head per work item                   */
  int heads_per_item;        /* query heads of one key/value head per work item     */
  int keys_per_tile;         /* keys per tile                                       */
  int kernel;                /* 0 = fp32 kernel, 1 = bf16 matrix-core kernel,
                                2 = FP8 matrix-core kernel                           */
} attn_plan_info;

/* Fills *info for the given arguments; returns the same status attn_fwd would
 * return for them (pointers are not needed and not checked). */
int attn_plan(int B, int Hq, int Hkv, int S, int D, int mask_kind, int window,
              const int* global_idx, int n_global, int dtype, attn_plan_info* info);

/*
 * attn_decode -- enqueue decode attention of the Sq newest positions of every
 * sequence against its key/value cache on `stream`.
 *
 * Operation ("Trasformer 浅析", section 推理：KV 缓存: the output at step t is
 * the softmax of q_t against the cached keys of positions 1..t applied to the
 * cached values; "Transformer 架构及其变体", section 预填充创建缓存，解码复用缓存:
 * each step appends the new positions' keys and values to the cache, then the
 * new queries read the stored history; sequences may hold caches of
 * different lengths; "Transformer 演进与变体", section 稀疏注意力: under a
 * sliding window each position attends only to the last `window` positions
 * up to itself):
 *
 *   for every batch b, query head a, new position i < Sq:
 *     h   = a / (Hq / Hkv),   L = cache_len[b],   p_i = L - Sq + i
 *     visible positions j:  j <= p_i (ATTN_MASK_CAUSAL),  j < L (ATTN_MASK_FULL),
 *                           p_i - window < j <= p_i (ATTN_MASK_CAUSAL_WINDOW)
 *     o[b][a][i][:] = softmax_j(scale * q[b][a][i] . k[b][h][j]) applied to v[b][h][j][:]
 *
 *   q           device [B][Hq][Sq][D] bf16: queries of the Sq newest positions
 *   k_cache,    device [B][Hkv][Smax][D] bf16; sequence b's positions 0..L-1
 *   v_cache       hold its keys / values, including the Sq new ones (already
 *               appended); entries at or beyond L are never read into the result
 *   o           device [B][Hq][Sq][D] bf16, written; must not overlap the inputs
 *   cache_len   DEVICE pointer to B int32 lengths L in [0, Smax] (read by the
 *               kernel, so the call can be captured once and replayed with new
 *               lengths; values outside the range are clamped to it); NULL
 *               means every sequence holds Smax positions
 *   Sq          new positions per sequence, >= 1, with (Hq / Hkv) * Sq <= 32
 *               (all query rows of one key/value head share one matrix-core tile)
 *   Smax        cache capacity per sequence, >= 1
 *   D           head width, 64 or 128
 *   mask_kind   ATTN_MASK_CAUSAL, ATTN_MASK_FULL (identical when Sq == 1) or
 *               ATTN_MASK_CAUSAL_WINDOW (only the last window + Sq - 1
 *               positions of a sequence are read)
 *   window      >= 1 with ATTN_MASK_CAUSAL_WINDOW (a window of Smax or more
 *               is the causal mask), 0 otherwise; else ATTN_ERR_WINDOW
 *   scale       multiplies q.k, used exactly as given
 *   dtype       ATTN_DTYPE_BF16 (fp32 returns ATTN_ERR_UNSUPPORTED); arithmetic
 *               as for attn_fwd's bf16 path
 *   workspace   device scratch of at least the bytes attn_decode_workspace
 *               reports for the same arguments (NULL allowed when that is 0);
 *               16-byte aligned; owned by the caller, overwritten by the call;
 *               calls that may run at the same time need separate workspaces
 *
 * A query that sees no position (p_i < 0, or L == 0) is written as zeros.
 * The key ranges are cut into splits on the device from the lengths, in
 * proportion to each sequence's range (a long sequence takes more
 * workgroups than a short one).  Returns ATTN_OK after enqueuing one or two
 * kernels (the second merges key splits); no synchronisation, no allocation.
 * Argument errors are detected on the host before any launch.  Deterministic
 * for a given input and lengths.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                const int* cache_len, int B, int Hq, int Hkv, int Sq, int Smax, int D,
                int mask_kind, int window, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream);

/* Workspace bytes attn_decode needs for these arguments (0 when it needs
 * none); the same validation as attn_decode, no device access.  The size
 * depends on the shape, the mask and the window, not on the lengths or on
 * whether they are given: about 4.1 MiB (D = 128) or 2.1 MiB (D = 64) of
 * key-split partials plus 8 bytes per (sequence, key/value head) pair once a
 * sequence's key range can exceed 256 positions, else 0. */
int attn_decode_workspace(int B, int Hq, int Hkv, int Sq, int Smax, int D, int mask_kind,
                          int window, int dtype, size_t* workspace_bytes);

/* Bytes of the static device scratch behind attn_decode_noalloc (one array
 * per GPU the library runs on, held until the process ends). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory at all (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments, kernels and results as
 * attn_decode, without the workspace.  The key-split partials go to a static
 * device array of ATTN_NOALLOC_SCRATCH_BYTES per GPU instead; the call
 * allocates nothing (no hipMalloc, hipFree or allocating routine).
 *
 *   q, k_cache, v_cache, o, cache_len, B, Hq, Hkv, Sq, Smax, D, mask_kind,
 *   window, scale, dtype, stream   as for attn_decode
 *
 * The first call on a GPU looks up that GPU's copy of the array (with the
 * stream's device current for the lookup, restored afterwards).  Every call
 * on a GPU shares that array and leaves the last call's partials in it:
 * calls that may overlap on one GPU race and must be serialised by the
 * caller (one stream, or events).  Returns ATTN_ERR_SCRATCH, before any
 * launch, when attn_decode_workspace reports more than
 * ATTN_NOALLOC_SCRATCH_BYTES for the arguments (more than about a million
 * (sequence, key/value head) pairs), ATTN_ERR_HIP when the lookup fails,
 * otherwise the status attn_decode would return.
 */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                        const int* cache_len, int B, int Hq, int Hkv, int Sq, int Smax, int D,
                        int mask_kind, int window, float scale, int dtype, void* stream);

/* Static, NUL-terminated name of a status code. */
const char* attn_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
