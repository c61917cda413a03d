// milo_encode.cpp -- host side of the encode ABI declared in
// include/milo_encode.h: argument validation (before any HIP call),
// workspace sizing, the host-side pool layout and kernel launches on the
// caller's stream.  No allocation, no synchronisation, no global state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "kernels.h"
#include "milo_encode.h"

namespace {

constexpr size_t kEncWsAlign = 256;

inline size_t enc_round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool enc_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t n_mats(const milo_encode_args* a) { return (int64_t)a->n_blocks * a->n_kv_heads * 2; }

milo_status check_shape(const milo_encode_args* a) {
  if (!a) return MILO_ERR_INVALID;
  if (a->struct_size != (int32_t)sizeof(milo_encode_args)) return MILO_ERR_INVALID;
  if (a->dtype != MILO_F32 && a->dtype != MILO_BF16) return MILO_ERR_UNSUPPORTED;
  if (a->n_blocks < 0 || a->n_kv_heads < 1 || a->n_tokens < 0) return MILO_ERR_INVALID;
  if (a->head_dim != 64 && a->head_dim != 128) return MILO_ERR_UNSUPPORTED;
  if (n_mats(a) > INT32_MAX) return MILO_ERR_UNSUPPORTED;   // one workgroup per matrix
  if ((int64_t)a->n_kv_heads * a->n_tokens * a->head_dim > INT64_MAX / 4) return MILO_ERR_UNSUPPORTED;
  return MILO_OK;
}

size_t workspace_of(const milo_encode_args* a) {
  return enc_round_up((size_t)n_mats(a) * a->head_dim * a->head_dim * sizeof(float), kEncWsAlign);
}

milo_status check_common(const milo_encode_args* a) {
  milo_status st = check_shape(a);
  if (st != MILO_OK || a->n_blocks == 0) return st;
  if (!a->tok_start || !a->blocks) return MILO_ERR_INVALID;
  if (!enc_aligned(a->tok_start, 8) || !enc_aligned(a->blocks, 8)) return MILO_ERR_INVALID;
  if (a->n_tokens > 0 && (!a->k || !a->v)) return MILO_ERR_INVALID;
  if ((a->k && !enc_aligned(a->k, 16)) || (a->v && !enc_aligned(a->v, 16))) return MILO_ERR_INVALID;
  if (!a->workspace || a->workspace_bytes < workspace_of(a)) return MILO_ERR_WORKSPACE;
  if (!enc_aligned(a->workspace, kEncWsAlign)) return MILO_ERR_WORKSPACE;
  return MILO_OK;
}

milo::EncodeParams params_of(const milo_encode_args* a) {
  milo::EncodeParams p{};
  p.k = a->k;
  p.v = a->v;
  p.tok_start = a->tok_start;
  p.blocks = a->blocks;
  p.sigma = a->sigma;
  p.iters = a->iters;
  p.vecs = static_cast<float*>(a->workspace);
  p.pool = a->pool;
  p.n_blocks = a->n_blocks;
  p.n_kv_heads = a->n_kv_heads;
  p.n_tokens = a->n_tokens;
  return p;
}

int32_t rank_units(const milo_rank_args* a) { return (a->head_dim - a->r_min) / a->unit; }

milo_status check_rank(const milo_rank_args* a) {
  if (!a) return MILO_ERR_INVALID;
  if (a->struct_size != (int32_t)sizeof(milo_rank_args)) return MILO_ERR_INVALID;
  if (a->n_blocks < 0 || a->n_kv_heads < 1 || a->unit < 1) return MILO_ERR_INVALID;
  if (a->head_dim != 64 && a->head_dim != 128) return MILO_ERR_UNSUPPORTED;
  if (a->r_min < 0 || a->r_min > a->head_dim) return MILO_ERR_INVALID;
  if ((int64_t)a->n_blocks * 2 * (rank_units(a) + 1) > INT32_MAX) return MILO_ERR_UNSUPPORTED;
  for (int32_t budget : {a->budget_k, a->budget_v}) {
    const int64_t extra = (int64_t)budget - (int64_t)a->n_blocks * a->r_min;
    if (extra < 0 || extra % a->unit != 0 || extra / a->unit > (int64_t)a->n_blocks * rank_units(a))
      return MILO_ERR_INVALID;
  }
  return MILO_OK;
}

size_t rank_workspace_of(const milo_rank_args* a) {
  return enc_round_up((size_t)2 * a->n_blocks * std::max(rank_units(a), 1) * sizeof(float), kEncWsAlign);
}

}  // namespace

extern "C" {

size_t milo_rank_workspace_bytes(const milo_rank_args* a) {
  if (check_rank(a) != MILO_OK) return 0;
  return rank_workspace_of(a);
}

milo_status milo_rank_allocate(const milo_rank_args* a, void* hip_stream) {
  milo_status st = check_rank(a);
  if (st != MILO_OK) return st;
  if (a->n_blocks == 0) return MILO_OK;
  if (!a->sigma || !a->ranks || !enc_aligned(a->sigma, 4) || !enc_aligned(a->ranks, 4)) return MILO_ERR_INVALID;
  if (a->entropy && !enc_aligned(a->entropy, 4)) return MILO_ERR_INVALID;
  if (!a->workspace || a->workspace_bytes < rank_workspace_of(a) || !enc_aligned(a->workspace, kEncWsAlign))
    return MILO_ERR_WORKSPACE;
  milo::RankParams p{};
  p.sigma = a->sigma;
  p.gains = static_cast<float*>(a->workspace);
  p.ranks = a->ranks;
  p.entropy = a->entropy;
  p.n_blocks = a->n_blocks;
  p.n_kv_heads = a->n_kv_heads;
  p.n_units = rank_units(a);
  p.r_min = a->r_min;
  p.unit = a->unit;
  p.k_units_k = ((int64_t)a->budget_k - (int64_t)a->n_blocks * a->r_min) / a->unit;
  p.k_units_v = ((int64_t)a->budget_v - (int64_t)a->n_blocks * a->r_min) / a->unit;
  milo::clear_stale_error();
  if (milo::launch_rank(p, a->head_dim, reinterpret_cast<hipStream_t>(hip_stream)) != hipSuccess)
    return MILO_ERR_DEVICE;
  return MILO_OK;
}

size_t milo_encode_workspace_bytes(const milo_encode_args* a) {
  if (check_shape(a) != MILO_OK) return 0;
  return workspace_of(a);
}

milo_status milo_encode_spectrum(const milo_encode_args* a, void* hip_stream) {
  milo_status st = check_common(a);
  if (st != MILO_OK) return st;
  if (a->n_blocks == 0) return MILO_OK;
  if ((a->sigma && !enc_aligned(a->sigma, 4)) || (a->iters && !enc_aligned(a->iters, 4)))
    return MILO_ERR_INVALID;
  const milo::EncodeParams p = params_of(a);
  milo::clear_stale_error();
  if (milo::launch_encode_spectrum(p, a->dtype, a->head_dim, reinterpret_cast<hipStream_t>(hip_stream)) !=
      hipSuccess)
    return MILO_ERR_DEVICE;
  return MILO_OK;
}

milo_status milo_encode_factors(const milo_encode_args* a, void* hip_stream) {
  milo_status st = check_common(a);
  if (st != MILO_OK) return st;
  if (a->n_blocks == 0) return MILO_OK;
  if (!a->pool || !enc_aligned(a->pool, 16)) return MILO_ERR_INVALID;
  const milo::EncodeParams p = params_of(a);
  milo::clear_stale_error();
  if (milo::launch_encode_factors(p, a->dtype, a->head_dim, reinterpret_cast<hipStream_t>(hip_stream)) !=
      hipSuccess)
    return MILO_ERR_DEVICE;
  return MILO_OK;
}

milo_status milo_encode_layout(const int32_t* n_tok, const int32_t* rank_k, const int32_t* rank_v,
                               int32_t n_blocks, int32_t n_kv_heads, int32_t head_dim,
                               milo_block* blocks_out, int64_t* pool_elems) {
  if (n_blocks < 0 || n_kv_heads < 1 || head_dim < 1 || head_dim % 8 != 0 || !pool_elems)
    return MILO_ERR_INVALID;
  if (n_blocks > 0 && (!n_tok || !rank_k || !rank_v || !blocks_out)) return MILO_ERR_INVALID;
  int64_t off = 0;
  for (int32_t b = 0; b < n_blocks; ++b) {
    if (n_tok[b] < 0 || n_tok[b] > INT32_MAX - 7) return MILO_ERR_INVALID;
    if (rank_k[b] < 0 || rank_k[b] > head_dim || rank_v[b] < 0 || rank_v[b] > head_dim)
      return MILO_ERR_INVALID;
    const int32_t ld = (n_tok[b] + 7) / 8 * 8;
    blocks_out[b].off = off;
    blocks_out[b].n_tok = n_tok[b];
    blocks_out[b].ld_tok = ld;
    blocks_out[b].rank_k = rank_k[b];
    blocks_out[b].rank_v = rank_v[b];
    off += (int64_t)n_kv_heads * (rank_k[b] + rank_v[b]) * ((int64_t)ld + head_dim);
  }
  *pool_elems = off;
  return MILO_OK;
}

milo_status milo_quant_layout(const milo_block* src_blocks, int32_t n_blocks, int32_t n_kv_heads,
                              int32_t head_dim, milo_block* blocks_out, int64_t* pool_bytes) {
  if (n_blocks < 0 || n_kv_heads < 1 || head_dim < 1 || head_dim % 8 != 0 || !pool_bytes) return MILO_ERR_INVALID;
  if (n_blocks > 0 && (!src_blocks || !blocks_out)) return MILO_ERR_INVALID;
  int64_t off = 0;
  for (int32_t b = 0; b < n_blocks; ++b) {
    const milo_block& s = src_blocks[b];
    if (s.n_tok < 0 || s.n_tok > INT32_MAX - 63) return MILO_ERR_INVALID;
    if (s.rank_k < 0 || s.rank_k > head_dim || s.rank_v < 0 || s.rank_v > head_dim) return MILO_ERR_INVALID;
    const int32_t ld = (s.n_tok + 63) / 64 * 64;
    const int64_t rows = (int64_t)s.rank_k + s.rank_v;
    blocks_out[b].off = off;
    blocks_out[b].n_tok = s.n_tok;
    blocks_out[b].ld_tok = ld;
    blocks_out[b].rank_k = s.rank_k;
    blocks_out[b].rank_v = s.rank_v;
    const int64_t rk16 = ((int64_t)s.rank_k + 15) / 16 * 16;
    off += (int64_t)n_kv_heads * ((int64_t)s.n_tok * rk16 + (int64_t)s.rank_v * ld + rows * 2 * head_dim +
                                  (8 * rows + 15) / 16 * 16);
  }
  *pool_bytes = off;
  return MILO_OK;
}

milo_status milo_kivi_layout(const milo_block* src_blocks, int32_t n_blocks, int32_t n_kv_heads, int32_t head_dim,
                             int32_t bits, milo_block* blocks_out, int64_t* pool_bytes) {
  if (n_blocks < 0 || n_kv_heads < 1 || head_dim < 1 || head_dim % 8 != 0 || !pool_bytes) return MILO_ERR_INVALID;
  if (bits != 4 && bits != 2) return MILO_ERR_INVALID;
  if (n_blocks > 0 && (!src_blocks || !blocks_out)) return MILO_ERR_INVALID;
  int64_t off = 0;
  for (int32_t b = 0; b < n_blocks; ++b) {
    const milo_block& s = src_blocks[b];
    if (s.n_tok < 0 || s.n_tok > INT32_MAX - 63) return MILO_ERR_INVALID;
    if (s.rank_k < 0 || s.rank_k > head_dim || s.rank_v < 0 || s.rank_v > head_dim) return MILO_ERR_INVALID;
    const int32_t ld = (s.n_tok + 63) / 64 * 64;
    blocks_out[b].off = off;
    blocks_out[b].n_tok = s.n_tok;
    blocks_out[b].ld_tok = ld;
    blocks_out[b].rank_k = s.rank_k;
    blocks_out[b].rank_v = s.rank_v;
    off += (int64_t)n_kv_heads * milo::kivi_head_bytes(ld / 64, s.rank_k, s.rank_v, head_dim, bits);
  }
  *pool_bytes = off;
  return MILO_OK;
}

milo_status milo_quantize_kivi(const milo_quant_args* a, int32_t bits, void* hip_stream) {
  if (!a) return MILO_ERR_INVALID;
  if (a->struct_size != (int32_t)sizeof(milo_quant_args)) return MILO_ERR_INVALID;
  if (bits != 4 && bits != 2) return MILO_ERR_INVALID;
  if (a->n_blocks < 0 || a->n_kv_heads < 1) return MILO_ERR_INVALID;
  if (a->head_dim != 64 && a->head_dim != 128) return MILO_ERR_UNSUPPORTED;
  if ((int64_t)a->n_blocks * a->n_kv_heads > INT32_MAX) return MILO_ERR_UNSUPPORTED;
  if (a->n_blocks == 0) return MILO_OK;
  if (!a->src_pool || !a->src_blocks || !a->dst_pool || !a->dst_blocks) return MILO_ERR_INVALID;
  if (!enc_aligned(a->src_pool, 16) || !enc_aligned(a->dst_pool, 16) || !enc_aligned(a->src_blocks, 8) ||
      !enc_aligned(a->dst_blocks, 8))
    return MILO_ERR_INVALID;
  milo::QuantParams p{};
  p.src_pool = static_cast<const uint16_t*>(a->src_pool);
  p.src_blocks = a->src_blocks;
  p.dst_pool = static_cast<uint8_t*>(a->dst_pool);
  p.dst_blocks = a->dst_blocks;
  p.n_blocks = a->n_blocks;
  p.n_kv_heads = a->n_kv_heads;
  milo::clear_stale_error();
  if (milo::launch_quantize_kivi(p, a->head_dim, bits, reinterpret_cast<hipStream_t>(hip_stream)) != hipSuccess)
    return MILO_ERR_DEVICE;
  return MILO_OK;
}

milo_status milo_quantize_factors(const milo_quant_args* a, void* hip_stream) {
  if (!a) return MILO_ERR_INVALID;
  if (a->struct_size != (int32_t)sizeof(milo_quant_args)) return MILO_ERR_INVALID;
  if (a->n_blocks < 0 || a->n_kv_heads < 1) return MILO_ERR_INVALID;
  if (a->head_dim != 64 && a->head_dim != 128) return MILO_ERR_UNSUPPORTED;
  if ((int64_t)a->n_blocks * a->n_kv_heads > INT32_MAX) return MILO_ERR_UNSUPPORTED;
  if (a->n_blocks == 0) return MILO_OK;
  if (!a->src_pool || !a->src_blocks || !a->dst_pool || !a->dst_blocks) return MILO_ERR_INVALID;
  if (!enc_aligned(a->src_pool, 16) || !enc_aligned(a->dst_pool, 16) || !enc_aligned(a->src_blocks, 8) ||
      !enc_aligned(a->dst_blocks, 8))
    return MILO_ERR_INVALID;
  milo::QuantParams p{};
  p.src_pool = static_cast<const uint16_t*>(a->src_pool);
  p.src_blocks = a->src_blocks;
  p.dst_pool = static_cast<uint8_t*>(a->dst_pool);
  p.dst_blocks = a->dst_blocks;
  p.n_blocks = a->n_blocks;
  p.n_kv_heads = a->n_kv_heads;
  milo::clear_stale_error();
  if (milo::launch_quantize(p, a->head_dim, reinterpret_cast<hipStream_t>(hip_stream)) != hipSuccess)
    return MILO_ERR_DEVICE;
  return MILO_OK;
}

}  // extern "C"
