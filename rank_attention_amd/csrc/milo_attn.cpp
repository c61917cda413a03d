// milo_attn.cpp -- host side of the C ABI declared in include/milo_attn.h:
// argument validation (before any HIP call), workspace sizing and kernel
// launches on the caller's stream.  No allocation, no synchronisation, no
// global mutable state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "kernels.h"
#include "milo_attn.h"

namespace {

using milo::DecodeParams;
using milo::MergeParams;
using milo::Partials;

constexpr size_t kWsAlign = 256;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The caller's timing events (both or neither), stamped by the attention
// kernel's dispatch.
milo::LaunchEvents timing_events(const milo_attn_args* a) {
  milo::LaunchEvents ev;
  if (a->prof_events[0] && a->prof_events[1]) {
    ev.start = reinterpret_cast<hipEvent_t>(a->prof_events[0]);
    ev.stop = reinterpret_cast<hipEvent_t>(a->prof_events[1]);
  }
  return ev;
}

// Shape-only checks shared by the workspace query and the entry points.
milo_status check_shape(const milo_attn_args* a, int32_t path) {
  if (!a) return MILO_ERR_INVALID;
  if (a->struct_size != (int32_t)sizeof(milo_attn_args)) return MILO_ERR_INVALID;
  if (path != MILO_PATH_DECODE && path != MILO_PATH_CHUNK && path != MILO_PATH_SHARED) return MILO_ERR_INVALID;
  if (a->dtype != MILO_F32 && a->dtype != MILO_BF16 && a->dtype != MILO_BF16_Q8 && a->dtype != MILO_BF16_KV4 &&
      a->dtype != MILO_BF16_KV2)
    return MILO_ERR_UNSUPPORTED;
  if (a->batch < 0 || a->q_len < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1) return MILO_ERR_INVALID;
  if (a->n_q_heads % a->n_kv_heads != 0) return MILO_ERR_INVALID;
  if (a->max_blocks_per_seq < 0 || a->tail_cap < 0) return MILO_ERR_INVALID;
  if (!std::isfinite(a->scale)) return MILO_ERR_INVALID;
  if ((path == MILO_PATH_DECODE || path == MILO_PATH_SHARED) && a->q_len != 1) return MILO_ERR_INVALID;
  if (path == MILO_PATH_CHUNK && a->tail_cap < a->q_len) return MILO_ERR_INVALID;
  if (a->head_dim != 64 && a->head_dim != 128) return MILO_ERR_UNSUPPORTED;
  const int group = a->n_q_heads / a->n_kv_heads;
  // group sizes above 8 run on the MFMA kernel (bf16 storage)
  if (group > 16) return MILO_ERR_UNSUPPORTED;
  if (group > 8 && a->dtype != MILO_BF16) return MILO_ERR_UNSUPPORTED;
  // partial records (query rows x unit slots, up to 8 tail slots) are indexed in 32 bits on the device
  if ((int64_t)a->batch * a->q_len * a->n_q_heads * ((int64_t)a->max_blocks_per_seq + 8) > INT32_MAX)
    return MILO_ERR_UNSUPPORTED;
  // the MFMA chunk kernel (chunk and shared paths) reads bf16 storage
  if (path != MILO_PATH_DECODE && a->dtype != MILO_BF16) return MILO_ERR_UNSUPPORTED;
  return MILO_OK;
}

constexpr int kChunkRowsPerTile = 128;   // query rows per chunk workgroup
constexpr int kChunkTargetUnits = 1024;  // aim for >= 4 workgroups per CU

struct ChunkSplit {
  int32_t n_qtiles, n_ranges, blocks_per_range;
};

// Split each (sequence, KV head) into 128-row query tiles and block ranges
// so that the grid has about kChunkTargetUnits workgroups.  With a shared
// context the batch's query rows form one sequence of batch * group rows.
ChunkSplit chunk_split(const milo_attn_args* a, bool shared = false) {
  ChunkSplit c{};
  const int64_t rows = (int64_t)(shared ? a->batch : a->q_len) * (a->n_q_heads / a->n_kv_heads);
  c.n_qtiles = (int32_t)((rows + kChunkRowsPerTile - 1) / kChunkRowsPerTile);
  const int64_t base = std::max<int64_t>(1, (int64_t)(shared ? 1 : a->batch) * a->n_kv_heads * c.n_qtiles);
  const int32_t mb = std::max(a->max_blocks_per_seq, 1);
  int32_t nr = (int32_t)std::min<int64_t>(mb, std::max<int64_t>(1, (kChunkTargetUnits + base - 1) / base));
  c.blocks_per_range = (mb + nr - 1) / nr;
  c.n_ranges = (mb + c.blocks_per_range - 1) / c.blocks_per_range;
  return c;
}

// A shared context spreads each sequence's dense tail over pieces of one
// 64-token tile (at most 8), each its own trailing workgroup and unit slot:
// the tails run after the block workgroups, and short pieces finish
// together instead of one tail's whole length after the blocks.
int32_t shared_tail_pieces(const milo_attn_args* a) {
  return a->tail_cap > 0 ? std::min<int32_t>(8, (a->tail_cap + 63) / 64) : 1;
}

struct Layout {
  size_t o_bytes, ml_bytes, total;
  int64_t units;
  int32_t rows_per_unit;
  int32_t slots;
};

// Decode with more than 8 query heads per KV head runs on the MFMA kernel of
// the chunked path (q_len = 1: the whole tail is visible, as in decode); the
// vector-ALU decode kernel keeps G scores per token in registers.
bool decode_on_mfma(const milo_attn_args* a) { return a->n_q_heads / a->n_kv_heads > 8; }

Layout layout_of(const milo_attn_args* a, int32_t path) {
  Layout L{};
  const int group = a->n_q_heads / a->n_kv_heads;
  const bool ranges = path == MILO_PATH_CHUNK || (path == MILO_PATH_DECODE && decode_on_mfma(a));
  L.slots = ranges                     ? chunk_split(a).n_ranges + 1
            : path == MILO_PATH_SHARED ? chunk_split(a, true).n_ranges + shared_tail_pieces(a)
                                       : a->max_blocks_per_seq + 1;
  L.rows_per_unit = a->q_len * group;
  L.units = (int64_t)a->batch * a->n_kv_heads * L.slots;
  L.o_bytes = round_up((size_t)L.units * L.rows_per_unit * a->head_dim * sizeof(float), kWsAlign);
  L.ml_bytes = round_up((size_t)L.units * L.rows_per_unit * 2 * sizeof(float), kWsAlign);
  L.total = L.o_bytes + L.ml_bytes;
  return L;
}

milo_status check_pointers(const milo_attn_args* a, const Layout& L) {
  if (a->batch == 0) return MILO_OK;
  if (!a->q || !a->out || !a->seq_blocks) return MILO_ERR_INVALID;
  if (!aligned(a->q, 16) || !aligned(a->out, 16)) return MILO_ERR_INVALID;
  if (a->max_blocks_per_seq > 0) {
    if (!a->blocks || !a->pool) return MILO_ERR_INVALID;
    if (!aligned(a->pool, 16) || !aligned(a->blocks, 8)) return MILO_ERR_INVALID;
  }
  if ((a->tail_cap > 0) != (a->k_tail != nullptr) || (a->tail_cap > 0) != (a->v_tail != nullptr) ||
      (a->tail_cap > 0) != (a->tail_len != nullptr))
    return MILO_ERR_INVALID;
  if (a->tail_cap > 0 && (!aligned(a->k_tail, 16) || !aligned(a->v_tail, 16))) return MILO_ERR_INVALID;
  if (a->lse && !aligned(a->lse, 4)) return MILO_ERR_INVALID;
  if (!a->workspace || a->workspace_bytes < L.total) return MILO_ERR_WORKSPACE;
  if (!aligned(a->workspace, kWsAlign)) return MILO_ERR_WORKSPACE;
  return MILO_OK;
}

// The chunked path's launches (MFMA kernel, then the merge) with the
// partials at ws; q_len may be 1 (decode with G > 8).
milo_status chunk_launch(const milo_attn_args* a, char* ws, hipStream_t stream) {
  const Layout L = layout_of(a, MILO_PATH_CHUNK);
  const int group = a->n_q_heads / a->n_kv_heads;
  const ChunkSplit cs = chunk_split(a);
  Partials part{reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + L.o_bytes)};

  milo::ChunkParams p{};
  p.q = a->q;
  p.pool = a->pool;
  p.blocks = a->blocks;
  p.seq_blocks = a->seq_blocks;
  p.k_tail = a->k_tail;
  p.v_tail = a->v_tail;
  p.tail_len = a->tail_len;
  p.part = part;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.n_q_heads = a->n_q_heads;
  p.n_kv_heads = a->n_kv_heads;
  p.max_blocks = a->max_blocks_per_seq;
  p.tail_cap = a->tail_cap;
  p.n_qtiles = cs.n_qtiles;
  p.n_ranges = cs.n_ranges;
  p.blocks_per_range = cs.blocks_per_range;
  p.part_rows = a->q_len * group;
  p.no_tail = 0;
  p.tail_pieces = 1;
  p.head_dim = a->head_dim;
  p.scale_log2 = a->scale * milo::kLog2eHost;

  milo::clear_stale_error();
  if (milo::launch_chunk(p, group, stream, timing_events(a)) != hipSuccess) return MILO_ERR_DEVICE;

  MergeParams m{};
  m.part = part;
  m.seq_blocks = a->seq_blocks;
  m.out = a->out;
  m.lse = a->lse;
  m.batch = a->batch;
  m.q_len = a->q_len;
  m.n_q_heads = a->n_q_heads;
  m.n_kv_heads = a->n_kv_heads;
  m.max_blocks = a->max_blocks_per_seq;
  m.slots = L.slots;
  m.rows_per_unit = L.rows_per_unit;
  m.tail_slot = cs.n_ranges;
  m.blocks_per_slot = cs.blocks_per_range;
  m.seq_stride = 1;
  if (milo::launch_merge(m, a->head_dim, stream) != hipSuccess) return MILO_ERR_DEVICE;
  return MILO_OK;
}

}  // namespace

namespace milo {

milo_status decode_check(const milo_attn_args* a, size_t* workspace_bytes) {
  milo_status st = check_shape(a, MILO_PATH_DECODE);
  if (st != MILO_OK) return st;
  const Layout L = layout_of(a, MILO_PATH_DECODE);
  *workspace_bytes = L.total;
  if (a->batch == 0) return MILO_OK;
  // every pointer rule but the workspace's
  milo_attn_args b = *a;
  b.workspace = reinterpret_cast<void*>(kWsAlign);
  b.workspace_bytes = L.total;
  return check_pointers(&b, L);
}

milo_status decode_launch(const milo_attn_args* a, void* workspace, void* hip_stream) {
  if (a->batch == 0) return MILO_OK;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  if (decode_on_mfma(a)) return chunk_launch(a, static_cast<char*>(workspace), stream);
  const Layout L = layout_of(a, MILO_PATH_DECODE);
  const int group = a->n_q_heads / a->n_kv_heads;
  char* ws = static_cast<char*>(workspace);
  Partials part{reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + L.o_bytes)};

  DecodeParams p{};
  p.q = a->q;
  p.pool = a->pool;
  p.blocks = a->blocks;
  p.seq_blocks = a->seq_blocks;
  p.k_tail = a->k_tail;
  p.v_tail = a->v_tail;
  p.tail_len = a->tail_len;
  p.part = part;
  p.batch = a->batch;
  p.n_q_heads = a->n_q_heads;
  p.n_kv_heads = a->n_kv_heads;
  p.max_blocks = a->max_blocks_per_seq;
  p.tail_cap = a->tail_cap;
  p.scale_log2 = a->scale * milo::kLog2eHost;
  p.unit_order = a->unit_order;

  milo::clear_stale_error();
  if (milo::launch_decode(p, a->dtype, a->head_dim, group, stream, timing_events(a)) != hipSuccess) return MILO_ERR_DEVICE;

  MergeParams m{};
  m.part = part;
  m.seq_blocks = a->seq_blocks;
  m.out = a->out;
  m.lse = a->lse;
  m.batch = a->batch;
  m.q_len = a->q_len;
  m.n_q_heads = a->n_q_heads;
  m.n_kv_heads = a->n_kv_heads;
  m.max_blocks = a->max_blocks_per_seq;
  m.slots = L.slots;
  m.rows_per_unit = L.rows_per_unit;
  m.tail_slot = a->max_blocks_per_seq;
  m.blocks_per_slot = 1;
  m.seq_stride = 1;
  if (milo::launch_merge(m, a->head_dim, stream) != hipSuccess) return MILO_ERR_DEVICE;
  return MILO_OK;
}

}  // namespace milo

extern "C" {

size_t milo_attn_workspace_bytes(const milo_attn_args* a, int32_t path) {
  if (check_shape(a, path) != MILO_OK) return 0;
  return layout_of(a, path).total;
}

milo_status milo_attn_decode(const milo_attn_args* a, void* hip_stream) {
  size_t need = 0;
  milo_status st = milo::decode_check(a, &need);
  if (st != MILO_OK) return st;
  if (a->batch > 0) {
    if (!a->workspace || a->workspace_bytes < need) return MILO_ERR_WORKSPACE;
    if (!aligned(a->workspace, kWsAlign)) return MILO_ERR_WORKSPACE;
  }
  return milo::decode_launch(a, a->workspace, hip_stream);
}

milo_status milo_attn_chunk(const milo_attn_args* a, void* hip_stream) {
  milo_status st = check_shape(a, MILO_PATH_CHUNK);
  if (st != MILO_OK) return st;
  const Layout L = layout_of(a, MILO_PATH_CHUNK);
  st = check_pointers(a, L);
  if (st != MILO_OK) return st;
  if (a->batch == 0) return MILO_OK;
  return chunk_launch(a, static_cast<char*>(a->workspace), reinterpret_cast<hipStream_t>(hip_stream));
}

milo_status milo_attn_decode_shared(const milo_attn_args* a, void* hip_stream) {
  milo_status st = check_shape(a, MILO_PATH_SHARED);
  if (st != MILO_OK) return st;
  const Layout L = layout_of(a, MILO_PATH_SHARED);
  st = check_pointers(a, L);
  if (st != MILO_OK) return st;
  if (a->batch == 0) return MILO_OK;

  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int group = a->n_q_heads / a->n_kv_heads;
  const ChunkSplit cs = chunk_split(a, true);
  char* ws = static_cast<char*>(a->workspace);
  Partials part{reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + L.o_bytes)};

  // One MFMA kernel launch.  Blocks: one "sequence" whose batch * group
  // query rows are the batch's queries (q is [batch][1][n_q_heads][d], the
  // same memory as [1][batch][n_q_heads][d]) over sequence 0's block list;
  // its partials land in every sequence's own unit slots (part_rows =
  // group).  Tails: batch * n_kv_heads trailing workgroups, each sequence's
  // own tail for its G rows, written to slot n_ranges of its units.
  milo::ChunkParams p{};
  p.q = a->q;
  p.pool = a->pool;
  p.blocks = a->blocks;
  p.seq_blocks = a->seq_blocks;
  p.k_tail = a->k_tail;
  p.v_tail = a->v_tail;
  p.tail_len = a->tail_len;
  p.part = part;
  p.batch = 1;
  p.q_len = a->batch;
  p.n_q_heads = a->n_q_heads;
  p.n_kv_heads = a->n_kv_heads;
  p.max_blocks = a->max_blocks_per_seq;
  p.tail_cap = a->tail_cap;
  p.n_qtiles = cs.n_qtiles;
  p.n_ranges = cs.n_ranges;
  p.blocks_per_range = cs.blocks_per_range;
  p.part_rows = group;
  p.no_tail = 1;
  p.tail_pieces = shared_tail_pieces(a);
  p.head_dim = a->head_dim;
  p.tail_units = a->batch * a->n_kv_heads * p.tail_pieces;
  p.scale_log2 = a->scale * milo::kLog2eHost;

  milo::clear_stale_error();
  if (milo::launch_chunk(p, group, stream, timing_events(a)) != hipSuccess) return MILO_ERR_DEVICE;

  MergeParams m{};
  m.part = part;
  m.seq_blocks = a->seq_blocks;
  m.out = a->out;
  m.lse = a->lse;
  m.batch = a->batch;
  m.q_len = 1;
  m.n_q_heads = a->n_q_heads;
  m.n_kv_heads = a->n_kv_heads;
  m.max_blocks = a->max_blocks_per_seq;
  m.slots = L.slots;
  m.rows_per_unit = L.rows_per_unit;
  m.tail_slot = cs.n_ranges;
  m.blocks_per_slot = cs.blocks_per_range;
  m.seq_stride = 0;                   // every sequence uses sequence 0's block count
  if (milo::launch_merge(m, a->head_dim, stream) != hipSuccess) return MILO_ERR_DEVICE;
  return MILO_OK;
}

milo_status milo_attn_validate(const milo_attn_args* a, int32_t path, int32_t n_descriptors,
                               int64_t pool_elems, uint64_t* status, void* hip_stream) {
  milo_status st = check_shape(a, path);
  if (st != MILO_OK) return st;
  if (n_descriptors < 0 || pool_elems < 0 || !status || !aligned(status, 8)) return MILO_ERR_INVALID;
  if (a->batch > 0 && !a->seq_blocks) return MILO_ERR_INVALID;
  if (n_descriptors > 0 && (!a->blocks || !aligned(a->blocks, 8))) return MILO_ERR_INVALID;
  if (a->tail_cap > 0 && !a->tail_len) return MILO_ERR_INVALID;
  milo::ValidateParams p{};
  p.blocks = a->blocks;
  p.seq_blocks = a->seq_blocks;
  p.tail_len = a->tail_len;
  p.status = reinterpret_cast<unsigned long long*>(status);
  p.pool_elems = pool_elems;
  p.n_descriptors = n_descriptors;
  p.n_seqs_checked = a->batch == 0 ? 0 : (path == MILO_PATH_SHARED ? 1 : a->batch);
  p.batch = a->batch;
  p.max_blocks = a->max_blocks_per_seq;
  p.n_kv_heads = a->n_kv_heads;
  p.head_dim = a->head_dim;
  p.tail_cap = a->tail_cap;
  p.tail_min = path == MILO_PATH_CHUNK ? a->q_len : 0;
  p.dtype = a->dtype;
  if (a->unit_order) {
    // the schedule's permutation check counts units in the call's workspace
    p.n_units = milo::decode_units(a->batch, a->n_kv_heads, a->max_blocks_per_seq);
    if (!a->workspace || !aligned(a->workspace, kWsAlign) || a->workspace_bytes < (size_t)p.n_units * 4)
      return MILO_ERR_WORKSPACE;
    p.unit_order = a->unit_order;
    p.unit_count = static_cast<unsigned*>(a->workspace);
  }
  milo::clear_stale_error();
  if (milo::launch_validate(p, reinterpret_cast<hipStream_t>(hip_stream)) != hipSuccess) return MILO_ERR_DEVICE;
  return MILO_OK;
}

milo_status milo_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                            void* hip_stream) {
  if (!buf || !sink || bytes % 16 != 0 || !aligned(buf, 16) || n_workgroups < 1) return MILO_ERR_INVALID;
  if (bytes == 0) return MILO_OK;
  milo::clear_stale_error();
  if (milo::launch_read_probe(buf, bytes, sink, n_workgroups, reinterpret_cast<hipStream_t>(hip_stream)) !=
      hipSuccess)
    return MILO_ERR_DEVICE;
  return MILO_OK;
}

milo_status milo_attn_plan_decode(const milo_block* blocks, int32_t n_descriptors,
                                  const int32_t* seq_blocks, const int32_t* tail_len, int32_t batch,
                                  int32_t n_kv_heads, int32_t max_blocks, int32_t head_dim,
                                  int32_t* order_out) {
  if (batch < 0 || n_kv_heads < 1 || max_blocks < 0 || head_dim < 1 || n_descriptors < 0) return MILO_ERR_INVALID;
  if (batch > 0 && (!seq_blocks || !order_out)) return MILO_ERR_INVALID;
  if (n_descriptors > 0 && !blocks) return MILO_ERR_INVALID;
  const int64_t slots = (int64_t)max_blocks + 1;
  const int64_t units = (int64_t)batch * n_kv_heads * slots;
  if (units > INT32_MAX) return MILO_ERR_UNSUPPORTED;   // unit indices are 32-bit
  // the host tables are read here, so their ranges are checked first: every
  // list lies inside the n_descriptors entries of blocks
  for (int32_t i = 0; i < batch; ++i)
    if (seq_blocks[i] < 0 || seq_blocks[i + 1] < seq_blocks[i] || seq_blocks[i + 1] > n_descriptors)
      return MILO_ERR_INVALID;
  // rank 0: dense-tail units (few, and per byte the slowest, so they go
  // first and never finish last); rank 1: block units, largest first;
  // rank 2: empty slots and empty tails
  std::vector<int64_t> cost((size_t)units, 0);
  std::vector<int8_t> rank((size_t)units, 2);
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t b0 = seq_blocks[i];
    const int32_t nb = std::min(seq_blocks[i + 1] - b0, max_blocks);
    for (int32_t g = 0; g < n_kv_heads; ++g) {
      const int64_t base = ((int64_t)i * n_kv_heads + g) * slots;
      for (int32_t s = 0; s < nb; ++s) {
        const milo_block& b = blocks[b0 + s];
        const int64_t r = std::max(b.rank_k, 0) + std::max(b.rank_v, 0);
        cost[(size_t)(base + s)] = r * ((int64_t)std::max(b.n_tok, 0) + head_dim);
        rank[(size_t)(base + s)] = 1;
      }
      const int64_t L = tail_len ? std::max(tail_len[i], 0) : 0;
      cost[(size_t)(base + max_blocks)] = 2 * L * head_dim;
      rank[(size_t)(base + max_blocks)] = L > 0 ? 0 : 2;
    }
  }
  std::vector<int32_t> idx((size_t)units);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
    if (rank[(size_t)x] != rank[(size_t)y]) return rank[(size_t)x] < rank[(size_t)y];
    return cost[(size_t)x] > cost[(size_t)y];
  });
  std::copy(idx.begin(), idx.end(), order_out);
  return MILO_OK;
}

const char* milo_status_str(milo_status s) {
  switch (s) {
    case MILO_OK: return "ok";
    case MILO_ERR_INVALID: return "invalid argument";
    case MILO_ERR_UNSUPPORTED: return "unsupported configuration";
    case MILO_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MILO_ERR_DEVICE: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t milo_abi_version(void) { return MILO_ABI_VERSION; }

}  // extern "C"
