// chunk.hip -- gfx950 chunked-query attention over a block-wise low-rank KV
// cache (MFMA path).
//
// MILO (summary at paperlayer.ai/abs/2609.29913v1) keeps each block's keys and
// values as separate low-rank factors K_b ~= U_b W_b, V_b ~= U'_b W'_b ("4.2
// Block-wise Low-Rank Compression") and attends over the selected blocks
// ("4.4 MILO Workflow").  With Q new query tokens per sequence the G heads of
// a KV group give M = Q*G query rows, and each block is a chain of dense
// contractions, evaluated here in the transposed absorbed order
//     P^T = W Q^T            (r x M)     scaled by scale*log2(e)
//     S^T = U P^T            (T x M)     scores, log2 units
//     E^T = exp2(S^T - m)                online softmax per query row
//     Z^T = U'^T E^T         (r' x M)
//     O^T += W'^T Z^T        (d x M)
// on v_mfma_f32_32x32x16_bf16.  Each result tile is consumed as the next
// MFMA's operand straight from its accumulator registers: a 32x32 result
// holds, in lane l, column l%32 and rows {8a + 4(l/32) + b}, which is exactly
// an A/B operand whose K index runs over those rows.  The partner operand is
// read from LDS with the same K permutation: rank-major U^T and row-major W'
// through ds_read_b64_tr_b16 (a 16-lane transpose read), U'^T rows with plain
// 8-byte reads.  Every query row's softmax state lives in the lanes that own
// its column, so rescaling is lane-local.
//
// Work unit = one workgroup of four waves (one per SIMD): (sequence, KV head,
// 128 query rows, block range); wave w owns rows 32w..32w+31 of the tile.
// The last range slot is the dense causal tail.  Units write (o~, m, l)
// partials that the merge kernel combines.  The query tiles that share a
// block range are given consecutive workgroup slots on one XCD, so they run
// together and read the range's factors from that XCD's L2.
//
// Per block: W and W' are staged in LDS and P^T is built from W and Q (Q
// re-read from L2).  The block's token factors then pass through LDS in 64-token
// tiles of U^T and U'^T, double buffered: the next tile's global loads are
// issued before the current tile is computed and written to the other
// buffer after it.  Within a tile both 32-token score tiles are issued on
// the MFMA pipe before the first softmax, so exp2 work overlaps MFMA work.
//
// Softmax: the running max m enters the score MFMA as its initial
// accumulator (-m), so the scores arrive relative to m.  m is raised only
// when a score exceeds it by more than 2^8 (weights stay <= 256, exact
// enough in fp32 and bf16); O, Z and l are rescaled only then.
//
// Precision: P is split into bf16 hi + lo parts (two MFMAs per score step),
// so scores keep ~16 mantissa bits; e = exp2(s - m) and Z are rounded to
// bf16 once each (relative 2^-9, averaging out over tokens and ranks).
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kD = 128;            // head_dim of this kernel
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kTT = 64;            // tokens per staged tile
constexpr int kUPitch = kTT + 8;   // LDS row pitch (elements) of the U^T tile (transposing reads)
constexpr int kVPitch = kTT + 4;   // LDS row pitch of the U'^T tile (8-byte row reads)
constexpr int kWPitch = kD + 8;    // LDS row pitch of W' and of the tail V tile
constexpr int kMaxR = 128;
constexpr int kChunksPerRow = kTT / 8;                             // 16-byte chunks per tile row
constexpr int kStageSlots = 2 * kMaxR * kChunksPerRow / kThreads;  // chunks per thread per tile
constexpr float kRescaleGap = 8.f; // log2 units: weights may reach 2^8 before m moves

static_assert(kStageSlots * kThreads == 2 * kMaxR * kChunksPerRow, "tile staging split");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator register v for a lane in half kg: (v/4)*8 + 4kg + v%4.
__device__ __forceinline__ int acc_row(int v, int kg) { return (v >> 2) * 8 + 4 * kg + (v & 3); }

// 8 consecutive accumulator registers (8c .. 8c+7) as a bf16 operand, split
// into hi = bf16(x) and lo = bf16(x - hi).  Operands are assembled from
// packed 32-bit words only: per-element __bf16 inserts into a vector were
// lowered by hipcc (ROCm 7.2) to a broadcast of element 0.
__device__ __forceinline__ void split_operand(const f32x16_t& acc, int c, bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = acc[8 * c + 2 * k], x1 = acc[8 * c + 2 * k + 1];
    h[k] = pack_bf16(x0, x1);
    l[k] = pack_bf16(x0 - bf_lo(h[k]), x1 - bf_hi(h[k]));
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}
__device__ __forceinline__ bf16x8_t to_operand(const f32x16_t& acc, int c) {
  u32x4_t h;
#pragma unroll
  for (int k = 0; k < 4; ++k) h[k] = pack_bf16(acc[8 * c + 2 * k], acc[8 * c + 2 * k + 1]);
  return __builtin_bit_cast(bf16x8_t, h);
}

// Operand whose K index follows the accumulator row permutation, read from a
// K-major LDS array X (row = K index, pitch in elements, columns contiguous):
// slot s of lane l <- X[row0 + 4(l/32) + 8(s/4) + s%4][col0 + l%32].  Two
// transposing 8-byte reads per lane.  ds_read_b64_tr_b16 gives lane
// B + 4a + b (B = 16*(l/16)) element j = mem[addr(lane B + a + 4j) + b].
__device__ __forceinline__ bf16x8_t tr_operand(const uint16_t* X, int pitch, int row0, int col0,
                                               int lane) {
  const int kg = lane >> 5;
  const int r = row0 + 4 * kg + ((lane & 15) >> 2);
  const int c = col0 + 4 * (lane & 3) + 16 * ((lane >> 4) & 1);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(X + r * pitch + c));
  const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(X + (r + 8) * pitch + c));
  const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
  const u32x4_t w = {w0[0], w0[1], w1[0], w1[1]};
  return __builtin_bit_cast(bf16x8_t, w);
}

// Operand read along rows of an LDS array X (row = M index, columns = K):
// slot s of lane l <- X[row0 + l%32][col0 + 4(l/32) + 8(s/4) + s%4], the
// K permutation of an accumulator-sourced partner.  Two 8-byte reads.
__device__ __forceinline__ bf16x8_t row_operand(const uint16_t* X, int pitch, int row0, int col0,
                                                int lane) {
  const uint16_t* src = X + (row0 + (lane & 31)) * pitch + col0 + 4 * (lane >> 5);
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(src + 8);
  const u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8_t, w);
}

struct LdsLayout {
  uint16_t w[kMaxR * kWPitch];     // W (rank rows, zero-padded to a multiple of 32)
  uint16_t wp[kMaxR * kWPitch];    // W' (rank' rows, zero-padded to a multiple of 32)
  uint16_t u[2][kMaxR * kUPitch];  // U^T token tiles (double buffer); the tail's V tile
  uint16_t v[2][kMaxR * kVPitch];  // U'^T token tiles (double buffer)
};

// 16-byte load that yields zeros on lanes with !ok: their offset is pushed
// past the resource's size, and out-of-range raw buffer reads return 0, so
// no lane branches around the load.
__device__ __forceinline__ u32x4_t bld16_or0(rsrc_t rs, uint32_t off, bool ok) {
  return bld16(rs, ok ? off : 0x80000000u, 0);
}

// Stage rows [0, nrows_pad) x `chunks` 16-byte chunks of a row-major source
// (row stride src_ld elements, starting at byte offset base) into LDS with
// pitch `pitch`; rows >= nrows are written as zeros.
__device__ __forceinline__ void stage_rows(rsrc_t rs, uint32_t base, int src_ld, int nrows,
                                           int nrows_pad, int chunks, uint16_t* dst, int pitch,
                                           int tid) {
  for (int id = tid; id < nrows_pad * chunks; id += kThreads) {
    const int row = id / chunks, ch = id - row * chunks;
    const u32x4_t v = bld16_or0(rs, base + (uint32_t)(row * src_ld + ch * 8) * 2, row < nrows);
    *reinterpret_cast<u32x4_t*>(dst + row * pitch + ch * 8) = v;
  }
}

// One 64-token tile of a block: U^T rows [0, urows) then U'^T rows
// [0, vrows), 8 chunks of 16 bytes per row; chunk slot tid + kThreads*k.
// Rows past the rank are staged as zeros.
struct TileShape {
  int T, ld, r, rv, urows, vrows;
  uint32_t v_off;   // byte offset of U'^T in the head's factors
};

__device__ __forceinline__ void load_tile(u32x4_t (&pf)[kStageSlots], rsrc_t rs, const TileShape& s,
                                          int t0, int tid) {
#pragma unroll
  for (int k = 0; k < kStageSlots; ++k) {
    const int id = tid + kThreads * k;
    const bool is_u = id < s.urows * kChunksPerRow;
    const int id2 = is_u ? id : id - s.urows * kChunksPerRow;
    const int row = id2 / kChunksPerRow, tok = t0 + (id2 % kChunksPerRow) * 8;
    const bool ok = tok < s.ld && (is_u ? row < s.r : (row < s.rv && id2 < s.vrows * kChunksPerRow));
    pf[k] = bld16_or0(rs, (is_u ? 0u : s.v_off) + (uint32_t)(row * s.ld + tok) * 2, ok);
  }
}

// Write a loaded tile to LDS.  U'^T tokens >= T are zeroed (the pool's row
// padding may hold anything, and those columns meet e = 0 in the MFMA).
__device__ __forceinline__ void store_tile(const u32x4_t (&pf)[kStageSlots], uint16_t* U, uint16_t* V,
                                           const TileShape& s, int t0, int tid) {
#pragma unroll
  for (int k = 0; k < kStageSlots; ++k) {
    const int id = tid + kThreads * k;
    if (id < s.urows * kChunksPerRow) {
      const int row = id / kChunksPerRow, ch = id % kChunksPerRow;
      *reinterpret_cast<u32x4_t*>(U + row * kUPitch + ch * 8) = pf[k];
    } else if (id < (s.urows + s.vrows) * kChunksPerRow) {
      const int id2 = id - s.urows * kChunksPerRow;
      const int row = id2 / kChunksPerRow, ch = id2 % kChunksPerRow;
      u32x4_t v = pf[k];
      const int tok = t0 + ch * 8;
      if (tok + 8 > s.T) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          v[w] &= (tok + 2 * w < s.T ? 0xffffu : 0u) | (tok + 2 * w + 1 < s.T ? 0xffff0000u : 0u);
      }
      uint16_t* dst = V + row * kVPitch + ch * 8;
      *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{v[0], v[1]};
      *reinterpret_cast<u32x2_t*>(dst + 4) = u32x2_t{v[2], v[3]};
    }
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void milo_chunk_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) LdsLayout lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, kg = lane >> 5;

  // workgroup -> (sequence, KV head, range slot, query tile).  The grid holds
  // ceil(groups / 8) * 8 * n_qtiles workgroups, dispatched round-robin over
  // the 8 XCDs: slot k of XCD x runs query tile k % n_qtiles of group
  // (k / n_qtiles) * 8 + x.
  const int S = p.n_ranges + 1;
  const int n_groups = p.batch * p.n_kv_heads * S;
  const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
  const int group = (k8 / p.n_qtiles) * 8 + xcd;
  const int qt = k8 % p.n_qtiles;
  if (group >= n_groups) return;
  const int slot = group % S;
  const int g = (group / S) % p.n_kv_heads, i = group / (S * p.n_kv_heads);

  const int MQ = p.q_len * G;
  const int m0 = qt * (kWaves * kRowsPerWave) + wave * kRowsPerWave;
  const int m_l = m0 + (lane & 31);   // this lane's query row (column of every tile)
  const bool row_ok = m_l < MQ;
  const int j_l = m_l / G, hl = m_l - j_l * G;

  const int b0 = p.seq_blocks[i];
  const int nb = min(max(p.seq_blocks[i + 1] - b0, 0), p.max_blocks);
  const int blk_lo = slot * p.blocks_per_range;
  const int blk_hi = min(nb, blk_lo + p.blocks_per_range);
  const bool tail = slot == p.n_ranges;
  if (!tail && blk_lo >= blk_hi) return;   // empty range: the merge skips it

  // Q^T operand chunk kk: q[row m_l][16kk + 8kg .. +8], re-read (from L2)
  // where it is needed rather than held in registers.
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                         (((int64_t)i * p.q_len + (row_ok ? j_l : 0)) * p.n_q_heads + g * G +
                          (row_ok ? hl : 0)) * kD + 8 * kg;
  auto q_operand = [&](int kk) {
    u32x4_t v = {0, 0, 0, 0};
    if (row_ok) v = ld16(qrow + 16 * kk);
    return __builtin_bit_cast(bf16x8_t, v);
  };

  f32x16_t O[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[dt][v] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  // Reference the next score tile is taken relative to: the running max, or
  // 0 while this row has seen nothing.
  auto score_ref = [&]() { return m_run == kNegInf ? 0.f : m_run; };

  // Online softmax of one 32-token x 32-row score tile s whose entries are
  // s_true - mref (masked entries -inf).  Raises m when a score exceeds it
  // by more than kRescaleGap, rescaling O, Z and l, and returns
  // e = exp2(s_true - m) as two bf16 operands.
  auto softmax_tile = [&](f32x16_t& s, float mref, f32x16_t* Z, int nz, bf16x8_t (&eb)[2]) {
    float mx = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
    const bool need = mx + mref > m_run + kRescaleGap;
    if (__any(need)) {
      float a = mx + mref, b = mx + mref;
      swap32(a, b);
      const float m_new = fmaxf(m_run, fmaxf(a, b));
      const float alpha = (m_run == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) O[dt][v] *= alpha;
#pragma unroll
        for (int zt = 0; zt < kMaxR / 32; ++zt)
          if (zt < nz)
#pragma unroll
            for (int v = 0; v < 16; ++v) Z[zt][v] *= alpha;
        l_run *= alpha;
      }
      m_run = m_new;
    }
    const float shift = (m_run == kNegInf) ? 0.f : mref - m_run;
    if (__any(shift != 0.f)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] += shift;
    }
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float e = fast_exp2(s[v]);
      s[v] = e;
      sum += e;
    }
    l_run += sum;
    eb[0] = to_operand(s, 0);
    eb[1] = to_operand(s, 1);
  };

  if (!tail) {
    f32x16_t Z[kMaxR / 32];
    u32x4_t pf[kStageSlots];
    for (int b = blk_lo; b < blk_hi; ++b) {
      const milo_block blk = p.blocks[b0 + b];
      TileShape ts;
      ts.T = max(blk.n_tok, 0);
      ts.ld = blk.ld_tok;
      ts.r = min(max(blk.rank_k, 0), kD);
      ts.rv = min(max(blk.rank_v, 0), kD);
      const int r = ts.r, rv = ts.rv, T = ts.T;
      const int nrt = (r + 31) / 32, nvt = (rv + 31) / 32;
      ts.urows = nrt * 32;
      ts.vrows = nvt * 32;
      const uint16_t* head = reinterpret_cast<const uint16_t*>(p.pool) + blk.off +
                             (int64_t)g * (r + rv) * (ts.ld + kD);
      const rsrc_t rs = make_rsrc(head, (uint32_t)((r + rv) * (ts.ld + kD)) * 2);
      const uint32_t w_off = (uint32_t)(r * ts.ld) * 2;
      ts.v_off = w_off + (uint32_t)(r * kD) * 2;
      const uint32_t wp_off = ts.v_off + (uint32_t)(rv * ts.ld) * 2;
      const int ntiles = (T + kTT - 1) / kTT;

      __syncthreads();   // the previous block's LDS reads are done
      {
        // W and W' rows [0, 32*ceil(rank/32)) to LDS, all loads in flight together
        constexpr int kWSlots = kMaxR * (kD / 8) / kThreads;
        u32x4_t wv[kWSlots], wpv[kWSlots];
#pragma unroll
        for (int k = 0; k < kWSlots; ++k) {
          const int id = tid + kThreads * k, row = id / (kD / 8), ch = id % (kD / 8);
          const uint32_t off = (uint32_t)(row * kD + ch * 8) * 2;
          wv[k] = u32x4_t{0, 0, 0, 0};
          wpv[k] = u32x4_t{0, 0, 0, 0};
          if (row < ts.urows) wv[k] = bld16_or0(rs, w_off + off, row < r);
          if (row < ts.vrows) wpv[k] = bld16_or0(rs, wp_off + off, row < rv);
        }
#pragma unroll
        for (int k = 0; k < kWSlots; ++k) {
          const int id = tid + kThreads * k, row = id / (kD / 8), ch = id % (kD / 8);
          if (row < ts.urows) *reinterpret_cast<u32x4_t*>(lds.w + row * kWPitch + ch * 8) = wv[k];
          if (row < ts.vrows) *reinterpret_cast<u32x4_t*>(lds.wp + row * kWPitch + ch * 8) = wpv[k];
        }
      }
      if (ntiles > 0) load_tile(pf, rs, ts, 0, tid);
      __syncthreads();

      // ---- P^T = W Q^T per 32-rank tile, scaled, split into hi/lo operands
      bf16x8_t ph[kMaxR / 32][2], pl[kMaxR / 32][2];
#pragma unroll
      for (int rt = 0; rt < kMaxR / 32; ++rt) {
        if (rt < nrt) {
          f32x16_t acc;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] = 0.f;
          const uint16_t* wrow = lds.w + (32 * rt + (lane & 31)) * kWPitch + 8 * kg;
#pragma unroll
          for (int kk = 0; kk < kD / 16; ++kk) {
            const u32x4_t wa = *reinterpret_cast<const u32x4_t*>(wrow + 16 * kk);
            acc = mfma(__builtin_bit_cast(bf16x8_t, wa), q_operand(kk), acc);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acc[v] = (32 * rt + acc_row(v, kg) < r) ? acc[v] * p.scale_log2 : 0.f;
          split_operand(acc, 0, ph[rt][0], pl[rt][0]);
          split_operand(acc, 1, ph[rt][1], pl[rt][1]);
        }
      }
#pragma unroll
      for (int zt = 0; zt < kMaxR / 32; ++zt)
#pragma unroll
        for (int v = 0; v < 16; ++v) Z[zt][v] = 0.f;

      if (ntiles > 0) store_tile(pf, lds.u[0], lds.v[0], ts, 0, tid);
      __syncthreads();

      for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int t0 = t * kTT;
        if (t + 1 < ntiles) load_tile(pf, rs, ts, t0 + kTT, tid);
        const uint16_t* U = lds.u[buf];
        const uint16_t* V = lds.v[buf];

        // ---- S^T = U P^T (hi + lo) for both 32-token halves, issued together;
        // the accumulators start at -mref so scores arrive relative to it
        const float mref = score_ref();
        f32x16_t s[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[st][v] = -mref;
          if (t0 + 32 * st < T) {
#pragma unroll
            for (int rt = 0; rt < kMaxR / 32; ++rt) {
              if (rt < nrt) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                  if (32 * rt + 16 * c < r) {
                    const bf16x8_t a = tr_operand(U, kUPitch, 32 * rt + 16 * c, 32 * st, lane);
                    s[st] = mfma(a, ph[rt][c], s[st]);
                    s[st] = mfma(a, pl[rt][c], s[st]);
                  }
                }
              }
            }
          }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int tb = t0 + 32 * st;
          if (tb >= T) break;
          if (tb + 32 > T) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (tb + acc_row(v, kg) >= T) s[st][v] = kNegInf;
          }
          bf16x8_t eb[2];
          softmax_tile(s[st], mref, Z, nvt, eb);
          // ---- Z^T += U'^T E^T
#pragma unroll
          for (int vt = 0; vt < kMaxR / 32; ++vt) {
            if (vt < nvt) {
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const bf16x8_t a = row_operand(V, kVPitch, 32 * vt, 32 * st + 16 * c, lane);
                Z[vt] = mfma(a, eb[c], Z[vt]);
              }
            }
          }
        }
        if (t + 1 < ntiles) store_tile(pf, lds.u[buf ^ 1], lds.v[buf ^ 1], ts, t0 + kTT, tid);
        __syncthreads();
      }
      // ---- O^T += W'^T Z^T (W' staged and visible since the barriers above)
#pragma unroll
      for (int vt = 0; vt < kMaxR / 32; ++vt) {
        if (vt < nvt) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            if (32 * vt + 16 * c < rv) {
              const bf16x8_t zb = to_operand(Z[vt], c);
#pragma unroll
              for (int dt = 0; dt < kD / 32; ++dt) {
                const bf16x8_t a = tr_operand(lds.wp, kWPitch, 32 * vt + 16 * c, 32 * dt, lane);
                O[dt] = mfma(a, zb, O[dt]);
              }
            }
          }
        }
      }
    }
  } else {
    // ---- dense causal tail: token l is visible to query j iff l <= L - Q + j
    const int cap = p.tail_cap;
    const int L = min(max(p.tail_len[i], 0), cap);
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(p.k_tail) + ((size_t)i * p.n_kv_heads + g) * cap * kD;
    const uint16_t* vtp = reinterpret_cast<const uint16_t*>(p.v_tail) + ((size_t)i * p.n_kv_heads + g) * cap * kD;
    const rsrc_t rk = make_rsrc(kt, (uint32_t)(cap * kD) * 2);
    const rsrc_t rvv = make_rsrc(vtp, (uint32_t)(cap * kD) * 2);
    const int vis = L - p.q_len + j_l;   // last visible tail token of this row
    for (int t0 = 0; t0 < L; t0 += 32) {
      __syncthreads();
      stage_rows(rvv, (uint32_t)(t0 * kD) * 2, kD, min(32, L - t0), 32, kD / 8, lds.u[0], kWPitch, tid);
      __syncthreads();
      // S^T = K_tail q^T, K = d, taken relative to mref
      const float mref = score_ref();
      f32x16_t s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.f;
      const int krow = t0 + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) {
        const u32x4_t ka = bld16_or0(rk, (uint32_t)(krow * kD + 16 * kk + 8 * kg) * 2, krow < L);
        s = mfma(__builtin_bit_cast(bf16x8_t, ka), q_operand(kk), s);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + acc_row(v, kg);
        s[v] = (t < L && t <= vis) ? s[v] * p.scale_log2 - mref : kNegInf;
      }
      bf16x8_t eb[2];
      softmax_tile(s, mref, nullptr, 0, eb);
      // O^T += V_tail^T E^T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const bf16x8_t a = tr_operand(lds.u[0], kWPitch, 16 * c, 32 * dt, lane);
          O[dt] = mfma(a, eb[c], O[dt]);
        }
    }
  }

  // ---- partials: row m_l of this unit's record, o~ (d = 32dt + acc_row) and (m, l)
  {
    float a = l_run, b = l_run;
    swap32(a, b);
    l_run = a + b;
  }
  if (row_ok) {
    const size_t rec = ((size_t)((i * p.n_kv_heads + g) * S + slot)) * MQ + m_l;
    float* po = p.part.o + rec * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4_t*>(po + 32 * dt + q4 * 8 + 4 * kg) =
            f32x4_t{O[dt][4 * q4], O[dt][4 * q4 + 1], O[dt][4 * q4 + 2], O[dt][4 * q4 + 3]};
    if (kg == 0) {
      p.part.ml[rec * 2 + 0] = m_run;
      p.part.ml[rec * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_chunk(const ChunkParams& p, int group, hipStream_t s) {
  const int64_t groups = (int64_t)p.batch * p.n_kv_heads * (p.n_ranges + 1);
  if (groups == 0) return hipSuccess;
  const int64_t wgs = (groups + 7) / 8 * 8 * p.n_qtiles;
  const dim3 grid((unsigned)wgs), block(kThreads);
  switch (group) {
#define MILO_G(GG) \
  case GG: hipLaunchKernelGGL((milo_chunk_kernel<GG>), grid, block, 0, s, p); break;
    MILO_G(1) MILO_G(2) MILO_G(3) MILO_G(4) MILO_G(5) MILO_G(6) MILO_G(7) MILO_G(8)
#undef MILO_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace milo
