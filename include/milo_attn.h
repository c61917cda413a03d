/*
 * milo_attn.h -- C ABI of attention over a block-wise low-rank compressed KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * The method (MILO: Efficient Many-shot In-Context Learning with Block-wise
 * Low-rank Compression, summary at paperlayer.ai/abs/2609.29913v1):
 *  - the pre-encoded demonstration cache is split into blocks of several
 *    examples ("4.2 Block-wise Low-Rank Compression");
 *  - each block b keeps its keys and values separately as low-rank factors,
 *        K_b ~= U_b W_b      U_b: T_b x r_b,   W_b: r_b x d
 *        V_b ~= U'_b W'_b    U'_b: T_b x r'_b, W'_b: r'_b x d
 *    with block-specific ranks ("4.3 Dynamic Rank Allocation"), which may
 *    differ between keys and values ("4.4 MILO Workflow");
 *  - at inference the selected blocks are used for attention together
 *    ("4.4 MILO Workflow": retrieve selected blocks, reconstruct, attend).
 *
 * These entry points compute exactly that attention in the absorbed order
 * p = W_b q, s = scale * U_b p, one softmax over every listed block and a
 * dense recent-token tail, o = sum_b (a_b U'_b) W'_b + a_t V_t, without
 * materialising K_b or V_b.  For each query row (sequence i, position j,
 * query head h, KV head g = h / (n_q_heads / n_kv_heads)):
 *
 *   out[i][j][h] = sum_t softmax(s)_t v_t ,  lse[i][j][h] = log sum_t exp(s_t)
 *
 * over every token of every block listed for sequence i and the tail tokens
 * l < tail_len[i] - q_len + j + 1 (bottom-right causal; with q_len = 1 the
 * whole tail).  With nothing visible, out = 0 and lse = -inf.
 *
 * Conventions for every entry point:
 *  - all pointers in milo_attn_args are DEVICE pointers, except the args
 *    struct itself (host);  the caller owns every buffer;
 *  - calls are asynchronous on the given hipStream_t (NULL = default stream),
 *    never synchronise, never allocate and keep no pointer after returning;
 *  - host-checkable faults (null pointers, shapes, alignment, dtype, scale,
 *    workspace size) return a status before any HIP call and leave out/lse
 *    untouched;  a failed kernel launch returns MILO_ERR_DEVICE;
 *  - device-resident tables (blocks, seq_blocks, tail_len) are the caller's
 *    contract: ranks in [0, head_dim], n_tok >= 0, ld_tok >= n_tok and a
 *    multiple of 8, off a multiple of 8, every factor inside the pool,
 *    0 <= seq_blocks[i+1] - seq_blocks[i] <= max_blocks_per_seq (more are
 *    ignored), tail_len[i] in [0, tail_cap] (decode) or [q_len, tail_cap]
 *    (chunk).  Counts and lengths are clamped on the device;  offsets are not.
 *  - the library never prints, aborts or throws.
 */
#ifndef MILO_ATTN_H
#define MILO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MILO_ABI_VERSION 5

typedef enum milo_status {
  MILO_OK = 0,
  MILO_ERR_INVALID = 1,      /* null pointer, shape rule, misalignment, non-finite scale */
  MILO_ERR_UNSUPPORTED = 2,  /* well-formed but not built: head_dim, group size, dtype   */
  MILO_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required               */
  MILO_ERR_DEVICE = 4        /* a HIP call failed (launch error)                         */
} milo_status;

typedef enum milo_dtype {
  MILO_F32 = 0,              /* IEEE fp32 storage                                        */
  MILO_BF16 = 1,             /* bfloat16 storage                                         */
  MILO_BF16_Q8 = 2,          /* bfloat16 q, tail, W, W'; 8-bit token factors (decode)    */
  MILO_BF16_KV4 = 3,         /* bfloat16 q, tail, W, W'; KIVI-style 4-bit token factors
                                (decode)                                                 */
  MILO_BF16_KV2 = 4          /* the same with 2-bit codes                                */
} milo_dtype;

typedef enum milo_path {
  MILO_PATH_DECODE = 0,      /* one new query token per sequence                         */
  MILO_PATH_CHUNK = 1,       /* q_len new query tokens per sequence                      */
  MILO_PATH_SHARED = 2       /* one query token per sequence, one context for the batch  */
} milo_path;

/*
 * One compressed block, all KV heads (24 bytes, device memory).
 * KV head g's factors start at element  off + g * (rank_k + rank_v) * (ld_tok + head_dim)
 * of the pool and are laid out back to back:
 *     U^T  [rank_k][ld_tok]   keys' token factor, rank-major (row k = column k of U_b)
 *     W    [rank_k][head_dim]
 *     U'^T [rank_v][ld_tok]   values' token factor, rank-major
 *     W'   [rank_v][head_dim]
 * Elements n_tok..ld_tok-1 of each U^T / U'^T row are padding and are never
 * used (they may hold anything, NaN included).
 */
/*
 * MILO_BF16_Q8 pool (decode path only; built by milo_quantize_factors in
 * milo_encode.h).  MILO's cache combines with asymmetric INT8 quantisation
 * (summary page, "5.3 Performance Analysis"); here the token factors carry
 * it.  Every row k of U^T and of U'^T (one rank component over the block's
 * tokens) holds uint8 codes c with an fp32 pair (a_k, b_k):
 *     element = a_k * c + b_k.
 * The keys' codes are stored token-major (U, one row of rank_k codes per
 * token, padded to rk16 = rank_k rounded up to 16), the values' rank-major
 * (U'^T) in tiles of 64 tokens, the orders in which the decode kernel's
 * matrix-core operands take them.  Offsets and strides count BYTES: off is
 * a multiple of 16, ld_tok = n_tok rounded up to 64, and KV head g starts
 * at byte off + g * H with
 *     H = n_tok * rk16 + rank_v * ld_tok + 2 * (rank_k + rank_v) * head_dim
 *         + pad16(8 * (rank_k + rank_v)),
 * pad16(x) = x rounded up to a multiple of 16.  Per head, back to back:
 *     U codes     [n_tok][rk16]         uint8 (codes rank_k.. of a row: padding)
 *     W           [rank_k][head_dim]    bf16
 *     U'^T codes  [ld_tok/64][rank_v][64] uint8: token t of row k at byte
 *                 64 * (rank_v * (t / 64) + k) + t % 64 (tokens n_tok..: padding)
 *     W'          [rank_v][head_dim]    bf16
 *     (a_k, b_k)  [rank_k + rank_v][2]  fp32, the keys' rows first, then
 *                 padding to the next multiple of 16 bytes.
 * Padding codes may hold any value.
 */
/*
 * MILO_BF16_KV4 / MILO_BF16_KV2 pool (decode path only; built by
 * milo_quantize_kivi in milo_encode.h).  MILO's cache also combines with
 * KIVI quantisation (summary page, "5.3 Performance Analysis"): keys per
 * channel, values per token, asymmetric low-bit codes with an fp16 scale
 * and bias per group.  Here the token factors carry it (W and W' stay
 * bf16), with BITS = 4 or 2 and L = 2^BITS - 1:
 *   keys   U  (n_tok x rank_k): a group is one rank component k over the
 *          64 tokens of a chunk c (tokens 64c .. 64c+63 of the block);
 *   values U' (n_tok x rank_v): a group is one token t over 32 rank
 *          components (ranks 32v .. 32v+31);
 * element = a * code + b with the group's fp16 scale a and bias b.
 * Offsets and strides count BYTES: off is a multiple of 16, ld_tok = n_tok
 * rounded up to 64 (nch = ld_tok / 64 chunks), and with
 *     ng8 = ceil(rank_k / 8),  ngv = ceil(rank_v / 32),  ntv = ceil(rank_v / 16)
 * KV head g starts at byte off + g * H,
 *     H = 16 + nch * (32 ng8 + 64 BITS ng8 + 256 ngv + 128 BITS ntv)
 *         + 2 * head_dim * (rank_k + rank_v).
 * H must stay below 2^32 bytes (the decode kernel addresses a head's tables
 * with 32-bit offsets; at rank 128 that is about 28M tokens per block).
 * Per head, back to back:
 *     header  amax_k, amax_v (fp32: the largest key and value scale of the
 *             head), 8 zero bytes
 *     KA      [nch][8 ng8] fp16   key scales a (ranks rank_k..: 0)
 *     KB      [nch][8 ng8] fp16   key biases b
 *     KC      [nch][ng8][16][4]   key code words (see below)
 *     VA      [nch][ngv][64] fp16 value scales a' (token 64c + x; tokens
 *                                 n_tok..: 0)
 *     VB      [nch][ngv][64] fp16 value biases b'
 *     VC      [nch][ntv][64][2 BITS bytes]  value code words
 *     W       [rank_k][head_dim] bf16
 *     W'      [rank_v][head_dim] bf16
 * Code words hold 8 codes (a 4-bit word is 32 bits, a 2-bit word 16 bits)
 * in the order of the decode kernel's matrix-core operands.  Key word
 * (g8, col, m) of chunk c holds ranks 8 g8 + i (i = 0..7) of chunk token
 * 16 (col / 4) + 4 m + col % 4.  Value words of tile kt, lane l of chunk c
 * hold rank 16 kt + l % 16 at chunk tokens 16 (l / 16) + 8 s + i for two
 * 8-code words s = 0, 1.  Inside a 4-bit word, code i sits in nibble 2i
 * (i < 4) or 2 (i - 4) + 1 (i >= 4), bits 4 nibble .. +3.  2-bit words come
 * in pairs sharing one 32-bit word: the key words (g8, col, 2d) and
 * (g8, col, 2d + 1) form dword d, the value words s = 0, 1 form the lane's
 * dword; with P = 4 u + i / 2, code i of word u in {0, 1} sits at bits
 * 8 (2 (P % 2) + i % 2) + 2 (P / 2) .. +1.
 * Padding codes (ranks past rank_k, tokens past n_tok) may hold any value;
 * padding scales and biases are 0.
 */
typedef struct milo_block {
  int64_t off;      /* element offset of KV head 0's U^T; multiple of 8 (Q8, KV4,
                       KV2: bytes, multiple of 16)                                 */
  int32_t n_tok;    /* T_b >= 0                                                    */
  int32_t ld_tok;   /* row stride of U^T and U'^T in elements; >= n_tok, mult. of 8
                       (Q8, KV4, KV2: multiple of 64, see the layouts above)       */
  int32_t rank_k;   /* r_b  in [0, head_dim]                                       */
  int32_t rank_v;   /* r'_b in [0, head_dim]                                       */
} milo_block;

typedef struct milo_attn_args {
  int32_t struct_size;         /* sizeof(milo_attn_args)                                   */
  int32_t dtype;               /* milo_dtype of q, pool, k_tail, v_tail (MILO_BF16_Q8,
                                  MILO_BF16_KV4, MILO_BF16_KV2: decode only, group size
                                  <= 8, pool layouts above)                                */
  int32_t batch;               /* sequences, >= 0                                           */
  int32_t q_len;               /* query tokens per sequence: 1 (decode) or Q >= 1 (chunk)   */
  int32_t n_q_heads;           /* >= 1, multiple of n_kv_heads                              */
  int32_t n_kv_heads;          /* >= 1; group size n_q_heads / n_kv_heads in [1, 16]; above
                                  8 only with MILO_BF16 storage (decode then runs on the
                                  matrix-core kernel of the chunked path, and its
                                  workspace follows that path's layout)                     */
  int32_t head_dim;            /* 64 or 128                                                 */
  float scale;                 /* softmax scale (e.g. 1/sqrt(head_dim)); finite             */
  const void* q;               /* [batch][q_len][n_q_heads][head_dim], 16-B aligned         */
  const void* pool;            /* factor pool, 16-B aligned; may be NULL if no block listed */
  const milo_block* blocks;    /* descriptor table                                          */
  const int32_t* seq_blocks;   /* [batch+1] CSR: sequence i uses blocks[seq_blocks[i] ..
                                  seq_blocks[i+1]-1] (order irrelevant)                     */
  int32_t max_blocks_per_seq;  /* host-known bound on blocks per sequence, >= 0             */
  int32_t tail_cap;            /* tail capacity in tokens, >= 0 (chunk: >= q_len)           */
  const void* k_tail;          /* [batch][n_kv_heads][tail_cap][head_dim]; NULL iff cap 0   */
  const void* v_tail;          /* same shape, 16-B aligned                                  */
  const int32_t* tail_len;     /* [batch] visible tail tokens; NULL iff tail_cap == 0       */
  float* out;                  /* [batch][q_len][n_q_heads][head_dim] fp32, 16-B aligned    */
  float* lse;                  /* [batch][q_len][n_q_heads] fp32 natural-log; may be NULL   */
  void* workspace;             /* scratch of milo_attn_workspace_bytes(), 256-B aligned     */
  size_t workspace_bytes;
  void* prof_events[2];        /* optional hipEvent_t pair (created by the caller): when
                                  both are set, [0] and [1] take the start and end time
                                  of the call's main attention kernel, stamped by its
                                  dispatch (timing hook)                                    */
  const int32_t* unit_order;   /* optional device array: the order in which the decode
                                  kernel takes its work units (see milo_attn_plan_decode);
                                  NULL = natural order.  Must be a permutation of
                                  [0, batch * n_kv_heads * (max_blocks_per_seq + 1)).
                                  Only the decode path reads it.                            */
} milo_attn_args;

/* Workspace the given path needs for these arguments; 0 if the arguments are
 * invalid or unsupported (shape fields only; pointers are not inspected). */
size_t milo_attn_workspace_bytes(const milo_attn_args* args, int32_t path);

/* Decode: q_len must be 1.  One query token per sequence attends over its
 * listed blocks and its whole tail (tail_len[i] tokens).  Writes out and lse. */
milo_status milo_attn_decode(const milo_attn_args* args, void* hip_stream);

/* Chunked query: q_len = Q >= 1 new tokens per sequence, whose own keys and
 * values are the last Q entries of the tail; query j sees every block token
 * and tail tokens l <= tail_len[i] - Q + j.  Writes out and lse.  Runs on
 * the matrix cores: bf16 storage only (MILO_ERR_UNSUPPORTED otherwise),
 * head_dim 64 or 128. */
milo_status milo_attn_chunk(const milo_attn_args* args, void* hip_stream);

/* Decode over one compressed context shared by the whole batch: the
 * pre-encoded many-shot cache of one demonstration set ("1. Introduction")
 * serving many test queries.  Same arguments and result as milo_attn_decode
 * (q_len must be 1), except that every sequence attends to the blocks listed
 * for sequence 0 (blocks[seq_blocks[0] .. seq_blocks[1]-1]; the other
 * sequences' lists are not read) plus its own tail.  The shared factors are
 * read once for all batch * group query rows of a KV head: the blocks are
 * evaluated as dense contractions on the MFMA path, so this entry point
 * needs bf16 storage (MILO_ERR_UNSUPPORTED otherwise); head_dim 64 or 128.
 * The sequences' own tails are evaluated in the same kernel launch.
 * Workspace: milo_attn_workspace_bytes(args, MILO_PATH_SHARED). */
milo_status milo_attn_decode_shared(const milo_attn_args* args, void* hip_stream);

/*
 * Decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * milo_attn_decode with the same arguments and result, except that
 * args->workspace and args->workspace_bytes are ignored.  The split-K
 * partials go to a static device buffer of MILO_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the
 * call allocates nothing.  Calls needing more than that
 * (milo_attn_workspace_bytes(args, MILO_PATH_DECODE) >
 * MILO_NOALLOC_SCRATCH_BYTES) return MILO_ERR_WORKSPACE before any HIP call.
 * Every call on one GPU shares that GPU's buffer: calls that overlap on one
 * GPU (concurrent streams or threads) race and must be serialised by the
 * caller.  Stream-ordered calls on one stream are safe.
 */
#define MILO_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
milo_status milo_attn_decode_noalloc(const milo_attn_args* args, void* hip_stream);

/*
 * Host-side scheduler for the decode kernel.  Decode work unit
 *     u = (i * n_kv_heads + g) * (max_blocks_per_seq + 1) + slot
 * covers block slot `slot` of sequence i, KV head g (slot = max_blocks_per_seq
 * is the dense tail).  Units differ in size by up to the ratio of their ranks,
 * and one decode call runs about two units per wave slot of the GPU, so
 * starting the largest first keeps the last units short (longest-processing-
 * time-first).  The cost of a block unit is its factor bytes, (r + r')(T + d).
 * Dense-tail units with tail_len > 0 are placed before every block unit: they
 * are few and stream more slowly per byte, and started late they would be
 * the last to finish.
 *
 * blocks (n_descriptors entries), seq_blocks, tail_len are HOST copies of
 * the device tables (tail_len may be NULL when tail_cap is 0);  order_out (host) receives
 * batch * n_kv_heads * (max_blocks_per_seq + 1) unit indices: non-empty
 * tails (longest first), then block units (largest first), then empty slots
 * and empty tails; ties in natural order.  The cache is static across
 * decode steps, so the plan is computed once and copied to the device.
 * For sequence i it reads blocks[seq_blocks[i] .. seq_blocks[i] +
 * min(seq_blocks[i+1] - seq_blocks[i], max_blocks_per_seq)).
 * Returns MILO_ERR_INVALID on null pointers, negative sizes or a sequence
 * with seq_blocks[i] < 0, seq_blocks[i+1] < seq_blocks[i] or
 * seq_blocks[i+1] > n_descriptors (checked before any descriptor is read);
 * MILO_ERR_UNSUPPORTED when the unit count exceeds INT32_MAX.
 */
milo_status milo_attn_plan_decode(const milo_block* blocks, int32_t n_descriptors,
                                  const int32_t* seq_blocks, const int32_t* tail_len, int32_t batch,
                                  int32_t n_kv_heads, int32_t max_blocks_per_seq, int32_t head_dim,
                                  int32_t* order_out);

/*
 * Device-side check of the tables a call reads, for debugging callers: the
 * kernels clamp counts and lengths but trust offsets, ranks and the decode
 * schedule.  Reads only blocks[0 .. n_descriptors), seq_blocks, tail_len and
 * unit_order (never the pool), in up to three kernels on the stream, and
 * writes *status (device, 8 bytes):
 *     UINT64_MAX                          every rule holds;
 *     ((uint64_t)rule << 32) | index     otherwise, the smallest violated
 *                                         milo_table_rule and, for it, the
 *                                         smallest offending index (sequence
 *                                         for rules 1, 2, 7; schedule position
 *                                         for rule 8; descriptor else).
 * With path MILO_PATH_SHARED only sequence 0's list is checked (the other
 * lists are not read by that path).  pool_elems is the pool size in
 * elements.  Host-checkable faults return a status as for the other entry
 * points (status must be 8-byte aligned).  With MILO_BF16_Q8, MILO_BF16_KV4
 * and MILO_BF16_KV2, pool_elems counts bytes, rule 4 asks for ld_tok a multiple of 64 (and, for the
 * KIVI-style layouts, a KV head under 2^32 bytes) and rule 5 for off a multiple of 16.  When args->unit_order is set, rule 8 checks that it is a
 * permutation of the decode units; the check counts units in args->workspace
 * (256-B aligned, at least 4 bytes per unit, which a decode workspace always
 * has; its contents are overwritten) and returns MILO_ERR_WORKSPACE without it.
 */
typedef enum milo_table_rule {
  MILO_TABLE_SEQ_RANGE = 1,        /* seq_blocks[i] < 0, decreasing, or past n_descriptors        */
  MILO_TABLE_TOO_MANY_BLOCKS = 2,  /* seq_blocks[i+1] - seq_blocks[i] > max_blocks_per_seq        */
  MILO_TABLE_RANK = 3,             /* rank_k or rank_v outside [0, head_dim]                      */
  MILO_TABLE_TOKENS = 4,           /* n_tok < 0, ld_tok < n_tok, ld_tok not a multiple of 8 (64), or a KIVI-style head of 2^32 bytes or more */
  MILO_TABLE_OFFSET = 5,           /* off < 0 or not a multiple of 8                              */
  MILO_TABLE_POOL_BOUNDS = 6,      /* the block's factors end past pool_elems                     */
  MILO_TABLE_TAIL_LEN = 7,         /* tail_len[i] outside [0, tail_cap] (decode, shared) or
                                      [q_len, tail_cap] (chunk)                                   */
  MILO_TABLE_UNIT_ORDER = 8        /* unit_order[u] outside [0, units) or naming a unit that
                                      another entry also names (units = batch * n_kv_heads *
                                      (max_blocks_per_seq + 1))                                  */
} milo_table_rule;

milo_status milo_attn_validate(const milo_attn_args* args, int32_t path, int32_t n_descriptors,
                               int64_t pool_elems, uint64_t* status, void* hip_stream);

/* Measurement helper: streams `bytes` (a multiple of 16, 16-B aligned) of
 * device memory once with the decode kernel's load form (16-byte
 * non-temporal loads, a contiguous slice per wave; n_workgroups of 256
 * threads, e.g. 4096) and discards the data.  `sink` (device, n_workgroups
 * uint32) is written only if an improbable checksum occurs.  Timing it with
 * events gives the read rate this device reaches, a ceiling beside the
 * published HBM peak. */
milo_status milo_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                            void* hip_stream);

/* Static description of a status code. */
const char* milo_status_str(milo_status status);

/* MILO_ABI_VERSION of the built library. */
int32_t milo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MILO_ATTN_H */
