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
// on v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x16_bf16 for an odd 16-rank
// remainder).  Each result tile is consumed as the next MFMA's operand
// straight from its registers: a 16x16 result holds, in lane l, column l%16
// and rows 4(l/16) + v, so two stacked results form a K = 32 operand whose
// slot s carries row 4(l/16) + s%4 + 16(s/4).  The partner operand is read
// from LDS in that K order: rank-major U^T and row-major W' (and the tail's
// V) through ds_read_b64_tr_b16, a 16-lane transposing read in which lane
// 16q + 4a + b receives element e of the 8 bytes addressed by lane
// 16q + a + 4e; U'^T rows with plain 8-byte reads.  Every query row's
// softmax state lives in the four lanes that own its column.
//
// Work unit = one workgroup of eight waves, two per SIMD: (sequence, KV
// head, 128 query rows, block range); wave w owns rows 16w..16w+15.  The
// last range slot is the dense causal tail.  Units write (o~, m, l)
// partials that the merge kernel combines.  The query tiles that share a
// block range get consecutive workgroup slots on one XCD, so they run
// together and read the range's factors from that XCD's L2.
//
// Per block: W and W' are staged in LDS and P^T is built from W and Q (Q
// re-read from L2).  The block's token factors then pass through LDS in
// 64-token tiles of U^T and U'^T, double buffered: the next tile's global
// loads are issued before the current tile is computed and written to the
// other buffer after it.  The score chain is compiled per count of 16-rank
// chunks, so it is straight-line code.
//
// Softmax: the running max m enters the score MFMA as its initial
// accumulator (-m), so scores arrive relative to m.  m is raised only when
// a score exceeds it by more than 2^8 (weights stay <= 256, exact enough in
// fp32 and bf16); O, Z and l are rescaled only then.
//
// Precision: P and Z are split into bf16 hi + lo parts (two MFMAs each), so
// scores and the value projection keep ~16 mantissa bits; e = exp2(s - m) is
// rounded to bf16 once (relative 2^-9 per weight, averaging out over tokens).
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kD = 128;            // head_dim of this kernel
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerTile = kWaves * kRowsPerWave;
constexpr int kTT = 64;            // tokens per staged tile
// LDS row pitches (elements).  A transposing read touches 8 consecutive rows
// per 32 lanes, 32 bytes each: a pitch of 40 (U^T) or 72 (W, W') 4-byte banks
// modulo 64 puts those rows on disjoint banks.
constexpr int kUPitch = kTT + 16;  // U^T tile
constexpr int kVPitch = kTT + 8;   // U'^T tile (8-byte row reads: 36 banks keep 32 lanes disjoint)
constexpr int kWPitch = kD + 16;   // W, W' and the tail's K and V tiles
constexpr int kMaxR = 128;
constexpr int kChunksPerRow = kTT / 8;                             // 16-byte chunks per tile row
constexpr int kStageSlots = 2 * kMaxR * kChunksPerRow / kThreads;  // chunks per thread per tile
constexpr int kWSlots = kMaxR * (kD / 8) / kThreads;               // chunks per thread of W (or W')
constexpr float kRescaleGap = 8.f; // log2 units: weights may reach 2^8 before m moves

static_assert(kStageSlots * kThreads == 2 * kMaxR * kChunksPerRow, "tile staging split");
static_assert(kWSlots * kThreads == kMaxR * (kD / 8), "W staging split");
static_assert(kRowsPerTile == 128, "the host splits query rows in tiles of 128");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                   __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// Two stacked 16x16 results (rows 0-15 in x, 16-31 in y) as a K = 32 bf16
// operand, split into hi = bf16(v) and lo = bf16(v - hi).  Operands are
// assembled from packed 32-bit words only: per-element __bf16 inserts into
// a vector were lowered by hipcc (ROCm 7.2) to a broadcast of element 0.
__device__ __forceinline__ void split_pair(const f32x4_t& x, const f32x4_t& y, u32x4_t& hi, u32x4_t& lo) {
  hi[0] = pack_bf16(x[0], x[1]);
  hi[1] = pack_bf16(x[2], x[3]);
  hi[2] = pack_bf16(y[0], y[1]);
  hi[3] = pack_bf16(y[2], y[3]);
  lo[0] = pack_bf16(x[0] - bf_lo(hi[0]), x[1] - bf_hi(hi[0]));
  lo[1] = pack_bf16(x[2] - bf_lo(hi[1]), x[3] - bf_hi(hi[1]));
  lo[2] = pack_bf16(y[0] - bf_lo(hi[2]), y[1] - bf_hi(hi[2]));
  lo[3] = pack_bf16(y[2] - bf_lo(hi[3]), y[3] - bf_hi(hi[3]));
}
// One 16x16 result as a K = 16 operand, split hi + lo.
__device__ __forceinline__ void split_one(const f32x4_t& x, u32x2_t& hi, u32x2_t& lo) {
  hi[0] = pack_bf16(x[0], x[1]);
  hi[1] = pack_bf16(x[2], x[3]);
  lo[0] = pack_bf16(x[0] - bf_lo(hi[0]), x[1] - bf_hi(hi[0]));
  lo[1] = pack_bf16(x[2] - bf_lo(hi[1]), x[3] - bf_hi(hi[1]));
}
__device__ __forceinline__ u32x4_t pack_pair(const f32x4_t& x, const f32x4_t& y) {
  return u32x4_t{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(y[0], y[1]),
                 pack_bf16(y[2], y[3])};
}

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
__device__ __forceinline__ u32x2_t tr_read(const uint16_t* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

// K = 32 operand from a K-major LDS array X (row = K index, columns = M):
// slot s of lane l <- X[row0 + 4(l/16) + s%4 + 16(s/4)][col0 + l%16].
__device__ __forceinline__ u32x4_t tr_operand(const uint16_t* X, int pitch, int row0, int col0, int lane) {
  const int r = row0 + 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int c = col0 + 4 * (lane & 3);
  const u32x2_t a = tr_read(X + r * pitch + c), b = tr_read(X + (r + 16) * pitch + c);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}
// K = 16 operand: slot s of lane l <- X[row0 + 4(l/16) + s][col0 + l%16].
__device__ __forceinline__ u32x2_t tr_operand16(const uint16_t* X, int pitch, int row0, int col0, int lane) {
  const int r = row0 + 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int c = col0 + 4 * (lane & 3);
  return tr_read(X + r * pitch + c);
}
// K = 32 operand read along rows of an LDS array X (row = M index, columns = K):
// slot s of lane l <- X[row0 + l%16][col0 + 4(l/16) + s%4 + 16(s/4)].
__device__ __forceinline__ u32x4_t row_operand(const uint16_t* X, int pitch, int row0, int col0, int lane) {
  const uint16_t* src = X + (row0 + (lane & 15)) * pitch + col0 + 4 * (lane >> 4);
  const u32x2_t a = *reinterpret_cast<const u32x2_t*>(src);
  const u32x2_t b = *reinterpret_cast<const u32x2_t*>(src + 16);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

struct TileBuf {
  uint16_t u[kMaxR * kUPitch];     // U^T rows x 64 tokens
  uint16_t v[kMaxR * kVPitch];     // U'^T rows x 64 tokens
};
struct LdsLayout {
  uint16_t w[kMaxR * kWPitch];     // W rows (zero-padded to a multiple of 16); the tail's K tile
  uint16_t wp[kMaxR * kWPitch];    // W' rows (zero-padded to a multiple of 16); the tail's V tile
  TileBuf tile[2];                 // token tiles, double buffered
};

// 16-byte load that yields zeros on lanes with !ok: their offset is pushed
// past the resource's size, and out-of-range raw buffer reads return 0, so
// no lane branches around the load.
__device__ __forceinline__ u32x4_t bld16_or0(rsrc_t rs, uint32_t off, bool ok) {
  return bld16(rs, ok ? off : 0x80000000u, 0);
}

// One 64-token tile of a block: U^T rows [0, urows) then U'^T rows
// [0, vrows), 8 chunks of 16 bytes per row; this thread moves chunks
// tid + kThreads*k.  What does not change from tile to tile is worked out
// once per block: the chunk's byte offset in the factors (at token 0), its
// token offset, whether it is loaded at all (rows past the rank are staged
// as zeros) and where it lands in a tile buffer (-1: not staged).
struct StageSlots {
  uint32_t goff[kStageSlots];
  int tok[kStageSlots];
  int lds[kStageSlots];            // byte offset in TileBuf, or -1
  bool load[kStageSlots];
  bool is_v[kStageSlots];
};

__device__ __forceinline__ void plan_slots(StageSlots& ss, int tid, int r, int rv, int urows, int vrows,
                                           int ld, uint32_t v_off) {
#pragma unroll
  for (int k = 0; k < kStageSlots; ++k) {
    const int id = tid + kThreads * k;
    const bool is_u = id < urows * kChunksPerRow;
    const int id2 = is_u ? id : id - urows * kChunksPerRow;
    const int row = id2 / kChunksPerRow, ch = id2 % kChunksPerRow;
    const bool staged = is_u || id2 < vrows * kChunksPerRow;
    ss.tok[k] = ch * 8;
    ss.goff[k] = (is_u ? 0u : v_off) + (uint32_t)(row * ld + ch * 8) * 2;
    ss.load[k] = is_u ? row < r : (staged && row < rv);
    ss.is_v[k] = !is_u;
    ss.lds[k] = !staged ? -1
                        : (is_u ? (row * kUPitch + ch * 8) * 2
                                : (int)offsetof(TileBuf, v) + (row * kVPitch + ch * 8) * 2);
  }
}

__device__ __forceinline__ void load_tile(u32x4_t (&pf)[kStageSlots], rsrc_t rs, const StageSlots& ss,
                                          int ld, int t0) {
#pragma unroll
  for (int k = 0; k < kStageSlots; ++k)
    pf[k] = bld16_or0(rs, ss.goff[k] + (uint32_t)t0 * 2, ss.load[k] && t0 + ss.tok[k] < ld);
}

// Write a loaded tile to LDS.  U'^T tokens >= T are zeroed (the pool's row
// padding may hold anything, and those columns meet e = 0 in the MFMA).
__device__ __forceinline__ void store_tile(const u32x4_t (&pf)[kStageSlots], TileBuf* buf,
                                           const StageSlots& ss, int T, int t0) {
  char* base = reinterpret_cast<char*>(buf);
#pragma unroll
  for (int k = 0; k < kStageSlots; ++k) {
    if (ss.lds[k] < 0) continue;
    u32x4_t v = pf[k];
    const int tok = t0 + ss.tok[k];
    if (ss.is_v[k] && tok + 8 > T) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        v[w] &= (tok + 2 * w < T ? 0xffffu : 0u) | (tok + 2 * w + 1 < T ? 0xffff0000u : 0u);
    }
    *reinterpret_cast<u32x4_t*>(base + ss.lds[k]) = v;
  }
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

__global__ __launch_bounds__(kThreads) void milo_chunk_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) LdsLayout lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q4 = lane >> 4;
  const int G = p.group;

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
  const int m_l = qt * kRowsPerTile + wave * kRowsPerWave + (lane & 15);  // this lane's column
  const bool row_ok = m_l < MQ;
  const int j_l = m_l / G, hl = m_l - j_l * G;

  const int b0 = p.seq_blocks[i];
  const int nb = min(max(p.seq_blocks[i + 1] - b0, 0), p.max_blocks);
  const int blk_lo = slot * p.blocks_per_range;
  const int blk_hi = min(nb, blk_lo + p.blocks_per_range);
  const bool tail = slot == p.n_ranges;
  if (!tail && blk_lo >= blk_hi) return;   // empty range: the merge skips it

  // Q^T operand chunks qv[kk] = q[row m_l][32kk + 8(l/16) .. +8], re-read
  // (from L2) where needed rather than held in registers.  Lanes past the
  // last row read row 0 instead: their columns are never written out.
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                         (((int64_t)i * p.q_len + (row_ok ? j_l : 0)) * p.n_q_heads + g * G +
                          (row_ok ? hl : 0)) * kD + 8 * q4;
  auto load_q = [&](u32x4_t (&qv)[kD / 32]) {
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) qv[kk] = ld16(qrow + 32 * kk);
  };

  f32x4_t O[kD / 16];
#pragma unroll
  for (int dt = 0; dt < kD / 16; ++dt) O[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t Z[kMaxR / 16];
  float m_run = kNegInf, l_run = 0.f;

  // Reference the next score tiles are taken relative to: the running max,
  // or 0 while this row has seen nothing.
  auto score_ref = [&]() { return m_run == kNegInf ? 0.f : m_run; };

  // Online softmax of four 16-token x 16-row score tiles s (64 tokens)
  // whose entries are s_true - mref (masked entries -inf).  Raises m when a
  // score exceeds it by more than kRescaleGap, rescaling O, Z[0..nz) and l,
  // and returns e = exp2(s_true - m) as two K = 32 bf16 operands.
  auto softmax64 = [&](f32x4_t (&s)[4], float mref, int nz, u32x4_t (&eb)[2]) {
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[tt][v]);
    const bool need = mx + mref > m_run + kRescaleGap;
    if (__any(need)) {
      float a = mx + mref, b = a;
      swap16(a, b);
      float c = fmaxf(a, b), d = c;
      swap32(c, d);
      const float m_new = fmaxf(m_run, fmaxf(c, d));
      const float alpha = (m_run == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < kD / 16; ++dt) O[dt] *= alpha;
#pragma unroll
        for (int zt = 0; zt < kMaxR / 16; ++zt)
          if (zt < nz) Z[zt] *= alpha;
        l_run *= alpha;
      }
      m_run = m_new;
    }
    const float shift = (m_run == kNegInf) ? 0.f : mref - m_run;
    if (__any(shift != 0.f)) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) s[tt] += shift;
    }
    float sum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = fast_exp2(s[tt][v]);
        s[tt][v] = e;
        sum += e;
      }
    l_run += sum;
    eb[0] = pack_pair(s[0], s[1]);
    eb[1] = pack_pair(s[2], s[3]);
  };

  if (!tail) {
    u32x4_t pf[kStageSlots];
    for (int b = blk_lo; b < blk_hi; ++b) {
      const milo_block blk = p.blocks[b0 + b];
      const int T = max(blk.n_tok, 0), ld = blk.ld_tok;
      const int r = min(max(blk.rank_k, 0), kD), rv = min(max(blk.rank_v, 0), kD);
      // 16-rank chunks: scores use at least one (a rank-0 block scores 0
      // against zero-padded factors); values use none for rank' 0
      const int nk = max(1, (r + 15) / 16), nv = (rv + 15) / 16;
      const int urows = nk * 16, vrows = nv * 16;
      const uint16_t* head = reinterpret_cast<const uint16_t*>(p.pool) + blk.off +
                             (int64_t)g * (r + rv) * (ld + kD);
      const rsrc_t rs = make_rsrc(head, (uint32_t)((r + rv) * (ld + kD)) * 2);
      const uint32_t w_off = (uint32_t)(r * ld) * 2;
      const uint32_t v_off = w_off + (uint32_t)(r * kD) * 2;
      const uint32_t wp_off = v_off + (uint32_t)(rv * ld) * 2;
      const int ntiles = (T + kTT - 1) / kTT;
      StageSlots ss;
      plan_slots(ss, tid, r, rv, urows, vrows, ld, v_off);

      __syncthreads();   // the previous block's LDS reads are done
      {
        // W and W' rows to LDS, all loads in flight together
        u32x4_t wv[kWSlots], wpv[kWSlots];
#pragma unroll
        for (int k = 0; k < kWSlots; ++k) {
          const int id = tid + kThreads * k, row = id / (kD / 8), ch = id % (kD / 8);
          const uint32_t off = (uint32_t)(row * kD + ch * 8) * 2;
          wv[k] = bld16_or0(rs, w_off + off, row < r);
          wpv[k] = bld16_or0(rs, wp_off + off, row < rv);
        }
#pragma unroll
        for (int k = 0; k < kWSlots; ++k) {
          const int id = tid + kThreads * k, row = id / (kD / 8), ch = id % (kD / 8);
          if (row < urows) *reinterpret_cast<u32x4_t*>(lds.w + row * kWPitch + ch * 8) = wv[k];
          if (row < vrows) *reinterpret_cast<u32x4_t*>(lds.wp + row * kWPitch + ch * 8) = wpv[k];
        }
      }
      u32x4_t qv[kD / 32];
      load_q(qv);
      if (ntiles > 0) load_tile(pf, rs, ss, ld, 0);
      __syncthreads();
#pragma unroll
      for (int zt = 0; zt < kMaxR / 16; ++zt) Z[zt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // Everything that depends on the number of 16-rank score chunks is
      // compiled per count, so the MFMA chains are straight-line code.
      auto body = [&](auto nk_c) {
        constexpr int NK = decltype(nk_c)::value;
        constexpr int NK2 = NK / 2;           // K = 32 chunks
        constexpr bool REM = (NK & 1) != 0;   // trailing K = 16 chunk
        // ---- P^T = W Q^T per 16-rank tile, scaled, split into hi/lo operands
        u32x4_t ph[NK2 > 0 ? NK2 : 1], pl[NK2 > 0 ? NK2 : 1];
        u32x2_t ph16, pl16;
        {
          f32x4_t pt[NK];
#pragma unroll
          for (int rt = 0; rt < NK; ++rt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* wrow = lds.w + (16 * rt + (lane & 15)) * kWPitch + 8 * q4;
#pragma unroll
            for (int kk = 0; kk < kD / 32; ++kk)
              acc = mfma32(*reinterpret_cast<const u32x4_t*>(wrow + 32 * kk), qv[kk], acc);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[v] = (16 * rt + 4 * q4 + v < r) ? acc[v] * p.scale_log2 : 0.f;
            pt[rt] = acc;
          }
#pragma unroll
          for (int j = 0; j < NK2; ++j) split_pair(pt[2 * j], pt[2 * j + 1], ph[j], pl[j]);
          if (REM) split_one(pt[NK - 1], ph16, pl16);
        }

        if (ntiles > 0) store_tile(pf, &lds.tile[0], ss, T, 0);
        __syncthreads();

        for (int t = 0; t < ntiles; ++t) {
          const int buf = t & 1;
          const int t0 = t * kTT;
          if (t + 1 < ntiles) load_tile(pf, rs, ss, ld, t0 + kTT);
          const uint16_t* U = lds.tile[buf].u;
          const uint16_t* V = lds.tile[buf].v;

          // ---- S^T = U P^T (hi + lo) for the tile's four 16-token blocks;
          // the chains start from -mref, so scores arrive relative to it.
          const float mref = score_ref();
          const f32x4_t bias = {-mref, -mref, -mref, -mref};
          // Chunk-outer order: the four chains' operand reads for one rank
          // chunk are in flight together before their MFMAs.
          f32x4_t s[4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) s[tt] = bias;
#pragma unroll
          for (int j = 0; j < NK2; ++j) {
            u32x4_t a[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) a[tt] = tr_operand(U, kUPitch, 32 * j, 16 * tt, lane);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              s[tt] = mfma32(a[tt], ph[j], s[tt]);
              s[tt] = mfma32(a[tt], pl[j], s[tt]);
            }
          }
          if (REM) {
            u32x2_t a[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) a[tt] = tr_operand16(U, kUPitch, 32 * NK2, 16 * tt, lane);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              s[tt] = mfma16(a[tt], ph16, s[tt]);
              s[tt] = mfma16(a[tt], pl16, s[tt]);
            }
          }
          if (t0 + kTT > T) {   // tokens past the block end
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
              for (int v = 0; v < 4; ++v)
                if (t0 + 16 * tt + 4 * q4 + v >= T) s[tt][v] = kNegInf;
          }
          u32x4_t eb[2];
          softmax64(s, mref, nv, eb);
          // ---- Z^T += U'^T E^T
          // pairs of rank' tiles, four operand reads in flight
#pragma unroll
          for (int vt = 0; vt < kMaxR / 16; vt += 2) {
            if (vt < nv) {
              u32x4_t a[4];
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                a[c] = row_operand(V, kVPitch, 16 * vt, 32 * c, lane);
                a[2 + c] = row_operand(V, kVPitch, 16 * vt + 16, 32 * c, lane);
              }
#pragma unroll
              for (int c = 0; c < 2; ++c) Z[vt] = mfma32(a[c], eb[c], Z[vt]);
              if (vt + 1 < nv) {
#pragma unroll
                for (int c = 0; c < 2; ++c) Z[vt + 1] = mfma32(a[2 + c], eb[c], Z[vt + 1]);
              }
            }
          }
          if (t + 1 < ntiles) store_tile(pf, &lds.tile[buf ^ 1], ss, T, t0 + kTT);
          __syncthreads();
        }
      };
      switch (nk) {
        case 1: body(IntC<1>{}); break;
        case 2: body(IntC<2>{}); break;
        case 3: body(IntC<3>{}); break;
        case 4: body(IntC<4>{}); break;
        case 5: body(IntC<5>{}); break;
        case 6: body(IntC<6>{}); break;
        case 7: body(IntC<7>{}); break;
        default: body(IntC<8>{}); break;
      }

      // ---- O^T += W'^T Z^T (W' staged and visible since the barriers above;
      // its rows past rank' are zero, as are Z's)
#pragma unroll
      for (int j = 0; j < kMaxR / 32; ++j) {
        if (2 * j + 1 < nv) {
          u32x4_t zh, zl;
          split_pair(Z[2 * j], Z[2 * j + 1], zh, zl);
#pragma unroll
          for (int dt = 0; dt < kD / 16; ++dt) {
            const u32x4_t a = tr_operand(lds.wp, kWPitch, 32 * j, 16 * dt, lane);
            O[dt] = mfma32(a, zh, O[dt]);
            O[dt] = mfma32(a, zl, O[dt]);
          }
        } else if (2 * j < nv) {
          u32x2_t zh, zl;
          split_one(Z[2 * j], zh, zl);
#pragma unroll
          for (int dt = 0; dt < kD / 16; ++dt) {
            const u32x2_t a = tr_operand16(lds.wp, kWPitch, 32 * j, 16 * dt, lane);
            O[dt] = mfma16(a, zh, O[dt]);
            O[dt] = mfma16(a, zl, O[dt]);
          }
        }
      }
    }
  } else {
    // ---- dense causal tail: token l is visible to query j iff l <= L - Q + j.
    // 64-token tiles of K and V are staged in LDS (the W and W' regions).
    const int cap = p.tail_cap;
    const int L = min(max(p.tail_len[i], 0), cap);
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(p.k_tail) + ((size_t)i * p.n_kv_heads + g) * cap * kD;
    const uint16_t* vtp = reinterpret_cast<const uint16_t*>(p.v_tail) + ((size_t)i * p.n_kv_heads + g) * cap * kD;
    const rsrc_t rk = make_rsrc(kt, (uint32_t)(cap * kD) * 2);
    const rsrc_t rvv = make_rsrc(vtp, (uint32_t)(cap * kD) * 2);
    const int vis = L - p.q_len + j_l;   // last visible tail token of this row
    u32x4_t qv[kD / 32];
    load_q(qv);
    constexpr int kTailSlots = kTT * (kD / 8) / kThreads;
    for (int t0 = 0; t0 < L; t0 += kTT) {
      __syncthreads();
      {
        u32x4_t kv[kTailSlots], vv[kTailSlots];
#pragma unroll
        for (int k = 0; k < kTailSlots; ++k) {
          const int id = tid + kThreads * k, row = id / (kD / 8), ch = id % (kD / 8);
          const uint32_t off = (uint32_t)((t0 + row) * kD + ch * 8) * 2;
          kv[k] = bld16_or0(rk, off, t0 + row < L);
          vv[k] = bld16_or0(rvv, off, t0 + row < L);
        }
#pragma unroll
        for (int k = 0; k < kTailSlots; ++k) {
          const int id = tid + kThreads * k, row = id / (kD / 8), ch = id % (kD / 8);
          *reinterpret_cast<u32x4_t*>(lds.w + row * kWPitch + ch * 8) = kv[k];
          *reinterpret_cast<u32x4_t*>(lds.wp + row * kWPitch + ch * 8) = vv[k];
        }
      }
      __syncthreads();
      // S^T = K_tail q^T (K = d), scaled, relative to mref, causally masked
      const float mref = score_ref();
      f32x4_t s[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* krow = lds.w + (16 * tt + (lane & 15)) * kWPitch + 8 * q4;
#pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk)
          acc = mfma32(*reinterpret_cast<const u32x4_t*>(krow + 32 * kk), qv[kk], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = t0 + 16 * tt + 4 * q4 + v;
          acc[v] = (tok < L && tok <= vis) ? acc[v] * p.scale_log2 - mref : kNegInf;
        }
        s[tt] = acc;
      }
      u32x4_t eb[2];
      softmax64(s, mref, 0, eb);
      // O^T += V_tail^T E^T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < kD / 16; ++dt)
          O[dt] = mfma32(tr_operand(lds.wp, kWPitch, 32 * c, 16 * dt, lane), eb[c], O[dt]);
    }
  }

  // ---- partials: row m_l of this unit's record, o~ (d = 16dt + 4(l/16) + v) and (m, l)
  {
    float a = l_run, b = l_run;
    swap16(a, b);
    float c = a + b, d = c;
    swap32(c, d);
    l_run = c + d;
  }
  if (row_ok) {
    const size_t rec = ((size_t)((i * p.n_kv_heads + g) * S + slot)) * MQ + m_l;
    float* po = p.part.o + rec * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt)
      *reinterpret_cast<f32x4_t*>(po + 16 * dt + 4 * q4) = O[dt];
    if (q4 == 0) {
      p.part.ml[rec * 2 + 0] = m_run;
      p.part.ml[rec * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_chunk(const ChunkParams& p, int group, hipStream_t s) {
  const int64_t groups = (int64_t)p.batch * p.n_kv_heads * (p.n_ranges + 1);
  if (groups == 0) return hipSuccess;
  if (group < 1 || group > 8) return hipErrorInvalidValue;
  const int64_t wgs = (groups + 7) / 8 * 8 * p.n_qtiles;
  ChunkParams q = p;
  q.group = group;
  hipLaunchKernelGGL(milo_chunk_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, s, q);
  return hipGetLastError();
}

}  // namespace milo
