/*
 * milo_encode.h -- C ABI of the encode step that produces the factors
 * milo_attn.h attends over, for AMD Instinct MI355X (gfx950).
 *
 * MILO (summary at paperlayer.ai/abs/2609.29913v1) pre-encodes a many-shot
 * demonstration context, splits its cache into blocks ("4.4 MILO Workflow":
 * partition, analyse, store) and keeps each block's keys and values as
 * separate low-rank factors ("4.2 Block-wise Low-Rank Compression") at
 * block-specific ranks ("4.3 Dynamic Rank Allocation").  The factorisation
 * is the truncated SVD: for a block X (T x d) of keys or values,
 *     W = the r right singular vectors of the largest singular values (rows)
 *     U = X W^T
 * so U W is the best rank-r approximation of X in Frobenius norm.
 *
 * Two calls, so that ranks can be chosen from the spectra in between:
 *   milo_encode_spectrum   singular values of every (block, KV head, K/V),
 *                          and the sorted singular vectors kept in the
 *                          workspace;
 *   milo_encode_factors    U^T, W, U'^T, W' of every block written into the
 *                          pool at the descriptors' offsets and ranks.
 * milo_encode_layout (host) places blocks of given sizes and ranks in a pool.
 *
 * Conventions are those of milo_attn.h: device pointers except the args
 * struct, asynchronous on the given stream, no allocation, host-checkable
 * faults reported before any HIP call, device tables are the caller's
 * contract (tok_start[b] >= 0 and tok_start[b] + n_tok <= n_tokens; token
 * ranges are clamped on the device).  Inputs must be finite.
 */
#ifndef MILO_ENCODE_H
#define MILO_ENCODE_H

#include "milo_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct milo_encode_args {
  int32_t struct_size;         /* sizeof(milo_encode_args)                                  */
  int32_t dtype;               /* milo_dtype of k, v and the factors written                */
  int32_t n_blocks;            /* >= 0                                                      */
  int32_t n_kv_heads;          /* >= 1                                                      */
  int32_t head_dim;            /* 64 or 128                                                 */
  int32_t n_tokens;            /* tokens per KV head in k and v, >= 0                       */
  const void* k;               /* [n_kv_heads][n_tokens][head_dim] dense keys, 16-B aligned */
  const void* v;               /* same shape: dense values                                  */
  const int64_t* tok_start;    /* [n_blocks]: block b covers tokens tok_start[b] ..
                                  tok_start[b] + blocks[b].n_tok - 1                        */
  const milo_block* blocks;    /* [n_blocks] descriptors.  Spectrum call: n_tok.  Factors
                                  call: also off, ld_tok, rank_k, rank_v (pool layout of
                                  milo_attn.h)                                              */
  float* sigma;                /* [n_blocks][n_kv_heads][2][head_dim] singular values,
                                  descending, K then V; written by the spectrum call; may
                                  be NULL                                                   */
  int32_t* iters;              /* [n_blocks][n_kv_heads][2] implicit QL iterations of the
                                  spectrum call (0: already diagonal; negative: an
                                  eigenvalue did not converge within 30 iterations); may
                                  be NULL                                                   */
  void* pool;                  /* factor pool written by the factors call, 16-B aligned     */
  void* workspace;             /* milo_encode_workspace_bytes() bytes, 256-B aligned: the
                                  spectrum call writes it, the factors call reads it        */
  size_t workspace_bytes;
} milo_encode_args;

/* Workspace both calls need (singular vectors of every matrix: 4 * head_dim^2
 * bytes each); 0 if the shape fields are invalid or unsupported. */
size_t milo_encode_workspace_bytes(const milo_encode_args* args);

/* Spectra: per (block, KV head, K/V) the Gram matrix X^T X (fp32 sums of
 * exact products) and its eigen-decomposition in fp32: Householder
 * reduction to tridiagonal form, then implicit QL iterations with the
 * rotations accumulated into the Householder factor.  sigma_i =
 * sqrt(max(lambda_i, 0)).  Writes sigma, iters and the workspace. */
milo_status milo_encode_spectrum(const milo_encode_args* args, void* hip_stream);

/* Factors: for every block, KV head and K/V, W = the first rank rows of the
 * sorted singular vectors and U^T = W X^T (fp32 sums), stored in dtype
 * (bf16: round to nearest even); U^T rows are zero past n_tok up to ld_tok.
 * Needs the workspace of a spectrum call on the same k, v, tok_start and
 * blocks[].n_tok. */
milo_status milo_encode_factors(const milo_encode_args* args, void* hip_stream);

/* Host-side layout: descriptors for blocks of n_tok[b] tokens and ranks
 * (rank_k[b], rank_v[b]) placed back to back in a pool (ld_tok =
 * n_tok rounded up to 8; every offset a multiple of 8 elements).  All
 * pointers are HOST arrays; blocks_out receives n_blocks descriptors and
 * *pool_elems the pool size in elements.  MILO_ERR_INVALID on null pointers,
 * negative sizes or ranks outside [0, head_dim]. */
milo_status milo_encode_layout(const int32_t* n_tok, const int32_t* rank_k, const int32_t* rank_v,
                               int32_t n_blocks, int32_t n_kv_heads, int32_t head_dim,
                               milo_block* blocks_out, int64_t* pool_elems);

/*
 * Rank allocation ("4.3 Dynamic Rank Allocation"): under a fixed total
 * budget, every block starts at r_min and the remaining rank units of size
 * `unit` go one at a time to the block whose next unit has the largest
 * marginal gain; keys and values have separate budgets ("4.4 MILO
 * Workflow").  The pages leave the entropy and the gain open; the readings:
 *   p     = the block's normalised energy sigma_i^2 / sum_j sigma_j^2 per KV
 *           head, averaged over its heads and renormalised (heads without
 *           energy contribute nothing);
 *   H     = -sum p_i ln p_i, high for slowly decaying spectra;
 *   gain of the unit raising rank r to r + unit = H * (p_r + .. + p_{r+unit-1});
 *   ties go to the lowest block index.
 * The result is exactly that greedy's (gains are non-increasing within a
 * block, so its picks are the K largest gains), computed without a
 * sequential loop.  Ranks never exceed r_min + unit * floor((head_dim -
 * r_min) / unit).
 */
typedef struct milo_rank_args {
  int32_t struct_size;         /* sizeof(milo_rank_args)                                    */
  int32_t n_blocks;            /* >= 0                                                      */
  int32_t n_kv_heads;          /* >= 1                                                      */
  int32_t head_dim;            /* 64 or 128                                                 */
  int32_t budget_k;            /* sum of the key ranks over all blocks                      */
  int32_t budget_v;            /* sum of the value ranks                                    */
  int32_t r_min;               /* minimum rank per block, 0 <= r_min <= head_dim            */
  int32_t unit;                /* rank granularity >= 1; each budget must be n_blocks *
                                  r_min plus a whole number of units that fit               */
  const float* sigma;          /* [n_blocks][n_kv_heads][2][head_dim] singular values,
                                  finite, descending per head (milo_encode_spectrum)        */
  int32_t* ranks;              /* out: [n_blocks][2] (rank_k, rank_v)                        */
  float* entropy;              /* out: [n_blocks][2] H of keys and values; may be NULL      */
  void* workspace;             /* milo_rank_workspace_bytes() bytes, 256-B aligned          */
  size_t workspace_bytes;
} milo_rank_args;

/* Workspace (the unit gains); 0 if the arguments are invalid. */
size_t milo_rank_workspace_bytes(const milo_rank_args* args);

/* Ranks of every block for keys and values (two kernels on the stream). */
milo_status milo_rank_allocate(const milo_rank_args* args, void* hip_stream);

/*
 * 8-bit token factors ("5.3 Performance Analysis" of the summary page:
 * the low-rank cache combines with asymmetric INT8 quantisation).  The
 * pages fix neither the grouping nor the rounding; the reading: every row
 * of U^T and U'^T (one rank component over the block's tokens, so each
 * group holds one scale of the decaying spectrum) is quantised
 * asymmetrically over its n_tok elements x_t, in fp32:
 *     lo = min x,  a = (hi - lo) / 255 (hi = max x),  b = lo,
 *     c_t = min(max(round_half_even((x_t - lo) / a), 0), 255)   (0 when a = 0),
 * every operation correctly rounded; a row with n_tok = 0 gets a = b = 0.
 * W and W' are copied unchanged.  The result is the MILO_BF16_Q8 pool of
 * milo_attn.h, which milo_attn_decode reads.
 */
typedef struct milo_quant_args {
  int32_t struct_size;         /* sizeof(milo_quant_args)                                   */
  int32_t n_blocks;            /* >= 0                                                      */
  int32_t n_kv_heads;          /* >= 1                                                      */
  int32_t head_dim;            /* 64 or 128                                                 */
  const void* src_pool;        /* MILO_BF16 pool (milo_attn.h layout), 16-B aligned         */
  const milo_block* src_blocks;/* [n_blocks] its descriptors                                */
  void* dst_pool;              /* MILO_BF16_Q8 pool, 16-B aligned, milo_quant_layout bytes  */
  const milo_block* dst_blocks;/* [n_blocks] from milo_quant_layout on the same source
                                  descriptors (same n_tok and ranks)                        */
} milo_quant_args;

/* Host-side layout of the MILO_BF16_Q8 pool for the blocks src_blocks
 * (HOST array): the same n_tok and ranks, ld_tok = n_tok rounded up to 64,
 * blocks back to back from byte 0 in the given order.  blocks_out (host)
 * receives n_blocks descriptors and *pool_bytes the pool size.
 * MILO_ERR_INVALID on null pointers, negative sizes or ranks outside
 * [0, head_dim]. */
milo_status milo_quant_layout(const milo_block* src_blocks, int32_t n_blocks, int32_t n_kv_heads,
                              int32_t head_dim, milo_block* blocks_out, int64_t* pool_bytes);

/* Quantise every block of the source pool into the destination pool (one
 * kernel on the stream; padding codes are written as 0).
 * The source tables are the caller's contract as in milo_attn.h. */
milo_status milo_quantize_factors(const milo_quant_args* args, void* hip_stream);

/*
 * KIVI-style token factors ("5.3 Performance Analysis" of the summary page:
 * the low-rank cache combines with KIVI quantisation, keys per channel and
 * values per token).  The pages fix neither group sizes nor rounding; the
 * reading, with L = 2^bits - 1 and bits = 4 or 2: the keys' token factor U
 * is grouped per rank component over each 64-token chunk of the block, the
 * values' U' per token over each run of 32 rank components; every group of
 * elements x (bf16 values, in fp32) gets
 *     a = fp16((max x - min x) / L),  b = fp16(min x),
 *     code = min(max(round_half_even((x - b) / a), 0), L)   (0 when a = 0)
 * with each fp32 step correctly rounded and a, b taken at their fp16
 * values.  W and W' are copied unchanged.  The result is the MILO_BF16_KV4
 * or MILO_BF16_KV2 pool of milo_attn.h, which milo_attn_decode reads.
 * Scales overflow to infinity when a group's range exceeds L times the
 * largest fp16 value (65504); such factors are outside the format.
 */

/* Host-side layout of the KIVI-style pool (bits 4 or 2) for the blocks
 * src_blocks (HOST array): the same n_tok and ranks, ld_tok = n_tok rounded
 * up to 64, blocks back to back from byte 0 in the given order.  blocks_out
 * (host) receives n_blocks descriptors and *pool_bytes the pool size.
 * MILO_ERR_INVALID on null pointers, negative sizes, ranks outside
 * [0, head_dim] or bits other than 4 and 2. */
milo_status milo_kivi_layout(const milo_block* src_blocks, int32_t n_blocks, int32_t n_kv_heads,
                             int32_t head_dim, int32_t bits, milo_block* blocks_out, int64_t* pool_bytes);

/* Quantise every block of the source pool (args->src_*) into the KIVI-style
 * pool args->dst_pool laid out by milo_kivi_layout with the same bits (one
 * kernel on the stream; padding codes, scales and biases are written as 0).
 * MILO_ERR_INVALID for bits other than 4 and 2. */
milo_status milo_quantize_kivi(const milo_quant_args* args, int32_t bits, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MILO_ENCODE_H */
