// kernels.h -- launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "milo_attn.h"

namespace milo {

constexpr float kLog2eHost = 1.4426950408889634f;

// The launchers check their launches with hipGetLastError, which reports
// the last error of any HIP call on the thread, also a hipErrorNotReady left
// behind by another library's event or stream query.  The entry points call
// this first, so that the check sees only their own launches.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Partial results of one work unit for its rows: unnormalised output o~
// ([rows][head_dim]) and the pair (m, l) per row, m in log2 units.
struct Partials {
  float* o;    // [n_units][rows_per_unit][head_dim]
  float* ml;   // [n_units][rows_per_unit][2]
};

struct DecodeParams {
  const void* q;
  const void* pool;
  const milo_block* blocks;
  const int32_t* seq_blocks;
  const void* k_tail;
  const void* v_tail;
  const int32_t* tail_len;
  Partials part;
  const int32_t* unit_order;   // optional largest-first permutation of the units
  int32_t batch, n_q_heads, n_kv_heads, max_blocks, tail_cap;
  float scale_log2;   // scale * log2(e)
};

struct ChunkParams {
  const void* q;
  const void* pool;
  const milo_block* blocks;
  const int32_t* seq_blocks;
  const void* k_tail;
  const void* v_tail;
  const int32_t* tail_len;
  Partials part;
  int32_t batch, q_len, n_q_heads, n_kv_heads, max_blocks, tail_cap;
  int32_t n_qtiles;          // tiles of 128 query rows over q_len * group rows
  int32_t n_ranges;          // block ranges per (sequence, KV head); slot n_ranges = tail
  int32_t blocks_per_range;
  int32_t group;             // query heads per KV head (set by launch_chunk)
  // Partial records: query row m of a unit of sequence i goes to sequence
  // i + m / part_rows, row m % part_rows of that sequence's unit slot
  // (part_rows = q_len * group, or group when the query rows of a shared
  // context stack the batch's sequences).
  int32_t part_rows;
  int32_t no_tail;           // skip the tail slots of the range groups
  // Shared context: after the block workgroups the launch has one
  // workgroup per (sequence, KV head) of the shared batch, tail_units =
  // batch * n_kv_heads of them, each the dense tail of that sequence's own
  // G query rows (q_len 1); 0 otherwise.
  int32_t tail_units;
  // Slots n_ranges .. n_ranges + tail_pieces - 1 hold the dense tail: piece
  // k covers its tiles [k * tpp, (k + 1) * tpp) of 64 tokens, tpp =
  // ceil(ceil(tail_cap / 64) / tail_pieces).  1 unless a shared context
  // spreads each tail over several trailing workgroups.
  int32_t tail_pieces;
  // 64 or 128.  The kernel's tiles are 128 wide; with 64, W, W', q and the
  // tail rows are zero-padded to 128 in LDS and registers (exact).
  int32_t head_dim;
  float scale_log2;
};

struct MergeParams {
  Partials part;
  const int32_t* seq_blocks;
  float* out;
  float* lse;
  int32_t batch, q_len, n_q_heads, n_kv_heads, max_blocks;
  int32_t slots;            // work-unit slots per (sequence, KV head)
  int32_t rows_per_unit;    // query rows stored per unit slot (q_len * group)
  int32_t tail_slot;        // first slot of the dense tail (every slot from it on is a tail piece)
  int32_t blocks_per_slot;  // slot s < tail_slot holds blocks [s*bps, (s+1)*bps)
  int32_t seq_stride;       // sequence i's block count is read at seq_blocks[i * seq_stride]
};

// Encode step: one workgroup per matrix m = (b * n_kv_heads + g) * 2 + kv.
struct EncodeParams {
  const void* k;               // [n_kv_heads][n_tokens][head_dim]
  const void* v;
  const int64_t* tok_start;    // [n_blocks]
  const milo_block* blocks;    // [n_blocks]
  float* sigma;                // [n_mats][head_dim] descending, or null
  int32_t* iters;              // [n_mats] QL iterations (negative: not converged), or null
  float* vecs;                 // [n_mats][head_dim][head_dim] eigenvector rows, descending
  void* pool;
  int32_t n_blocks, n_kv_heads, n_tokens;
};
hipError_t launch_encode_spectrum(const EncodeParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_encode_factors(const EncodeParams& p, int dtype, int head_dim, hipStream_t s);

// Rank allocation: unit gains per (K/V, block) in the workspace, then one
// selection per K/V.
struct RankParams {
  const float* sigma;          // [n_blocks][n_kv_heads][2][head_dim]
  float* gains;                // [2][n_blocks][n_units]
  int32_t* ranks;              // [n_blocks][2]
  float* entropy;              // [n_blocks][2] or null
  int32_t n_blocks, n_kv_heads, n_units, r_min, unit;
  int64_t k_units_k, k_units_v;   // units to hand out above r_min
};
hipError_t launch_rank(const RankParams& p, int head_dim, hipStream_t s);

// Device table check (milo_attn_validate).
struct ValidateParams {
  const milo_block* blocks;
  const int32_t* seq_blocks;
  const int32_t* tail_len;
  unsigned long long* status;
  int64_t pool_elems;        // bytes for 8-bit factor storage
  int32_t n_descriptors, n_seqs_checked, batch, max_blocks, n_kv_heads, head_dim, tail_cap, tail_min;
  int32_t dtype;             // storage type; the 8-bit and KIVI-style pools count bytes,
                             // with offsets multiples of 16 and ld_tok multiples of 64
  // decode schedule check (unit_order non-null): n_units entries, and one
  // count per unit in caller scratch
  const int32_t* unit_order;
  unsigned* unit_count;
  int64_t n_units;
};

// 8-bit factors: one workgroup per (block, KV head) quantises its U^T and
// U'^T rows and copies W and W'.
struct QuantParams {
  const uint16_t* src_pool;
  const milo_block* src_blocks;
  uint8_t* dst_pool;
  const milo_block* dst_blocks;
  int32_t n_blocks, n_kv_heads;
};
hipError_t launch_quantize(const QuantParams& p, int head_dim, hipStream_t s);

// KIVI-style factors: one workgroup per (block, KV head) quantises its
// chunks (keys per rank component and 64-token chunk, values per token and
// 32 rank components) and copies W and W'.
hipError_t launch_quantize_kivi(const QuantParams& p, int head_dim, int bits, hipStream_t s);

// Bytes of one KV head of a KIVI-style block with nch 64-token chunks
// (bits 4 or 2; the layout of milo_attn.h).
__host__ __device__ inline int64_t kivi_head_bytes(int64_t nch, int64_t r, int64_t rv, int64_t d, int bits) {
  const int64_t ng8 = (r + 7) / 8, ngv = (rv + 31) / 32, ntv = (rv + 15) / 16;
  return 16 + nch * (32 * ng8 + 64 * bits * ng8 + 256 * ngv + 128 * bits * ntv) + 2 * d * (r + rv);
}
hipError_t launch_validate(const ValidateParams& p, hipStream_t s);

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int n_wg, hipStream_t s);

// Work units of the decode kernel: one per (sequence, KV head, block slot),
// plus one dense-tail unit per (sequence, KV head).
inline int64_t decode_units(int batch, int n_kv_heads, int max_blocks) {
  return (int64_t)batch * n_kv_heads * (max_blocks + 1);
}

// Optional timing events of a launch: when set, the runtime stamps them with
// the kernel dispatch's own start and end (no separate stream commands).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// One instantiation per (dtype, head_dim), each in its own translation unit.
hipError_t launch_decode_dt_0_64(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_0_128(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_1_64(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_1_128(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_2_64(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_2_128(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_3_64(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_3_128(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_4_64(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_decode_dt_4_128(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev = {});

inline hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int group,
                                hipStream_t s, LaunchEvents ev = {}) {
  if (dtype == MILO_F32 && head_dim == 64) return launch_decode_dt_0_64(p, group, s, ev);
  if (dtype == MILO_F32 && head_dim == 128) return launch_decode_dt_0_128(p, group, s, ev);
  if (dtype == MILO_BF16 && head_dim == 64) return launch_decode_dt_1_64(p, group, s, ev);
  if (dtype == MILO_BF16 && head_dim == 128) return launch_decode_dt_1_128(p, group, s, ev);
  if (dtype == MILO_BF16_Q8 && head_dim == 64) return launch_decode_dt_2_64(p, group, s, ev);
  if (dtype == MILO_BF16_Q8 && head_dim == 128) return launch_decode_dt_2_128(p, group, s, ev);
  if (dtype == MILO_BF16_KV4 && head_dim == 64) return launch_decode_dt_3_64(p, group, s, ev);
  if (dtype == MILO_BF16_KV4 && head_dim == 128) return launch_decode_dt_3_128(p, group, s, ev);
  if (dtype == MILO_BF16_KV2 && head_dim == 64) return launch_decode_dt_4_64(p, group, s, ev);
  if (dtype == MILO_BF16_KV2 && head_dim == 128) return launch_decode_dt_4_128(p, group, s, ev);
  return hipErrorInvalidValue;
}
hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t s);
hipError_t launch_chunk(const ChunkParams& p, int group, hipStream_t s, LaunchEvents ev = {});

// The decode entry point in two halves (milo_attn.cpp), shared by
// milo_attn_decode and its variant with library-owned scratch: every
// argument check but the workspace's, giving the workspace size the call
// needs (no HIP call); then the launches with the partials at `workspace`.
milo_status decode_check(const milo_attn_args* a, size_t* workspace_bytes);
milo_status decode_launch(const milo_attn_args* a, void* workspace, void* hip_stream);

}  // namespace milo
