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
// Data movement: every factor byte goes from HBM straight into LDS with
// buffer_load ... lds (16 bytes per lane; lanes out of range write zeros,
// which pads ranks and token tiles).  The block's tokens pass in 64-token
// tiles of U^T and U'^T through three LDS buffers, two tiles ahead of the
// compute, across block boundaries; W of the next block is loaded during
// the last tile of the current one and W' at the start of its own block.
// LDS rows are unpadded; 16-byte chunks are XOR-swizzled per row so that
// every read pattern below touches each bank once per 32 lanes.  Waits are
// explicit (s_waitcnt vmcnt + s_barrier), so loads stay in flight across
// barriers.  The score chain is compiled per count of 16-rank chunks, so it
// is straight-line code.
//
// Softmax: the running max m enters the score MFMA as its initial
// accumulator (-m), so scores arrive relative to m.  m is raised only when
// a score exceeds it by more than 2^8 (weights stay <= 256, exact enough in
// fp32 and bf16); O, Z and l are rescaled only then.
//
// Precision: P and Z are split into bf16 hi + lo parts (two MFMAs each), so
// scores and the value projection keep ~16 mantissa bits; e = exp2(s - m) is
// rounded to bf16 once (relative 2^-9 per weight, averaging out over tokens).
#include <hip/hip_ext.h>

#include "device_common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace milo {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kD = 128;            // head_dim of this kernel
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerTile = kWaves * kRowsPerWave;
constexpr int kTT = 64;            // tokens per staged tile
constexpr int kMaxR = 128;
constexpr int kNBuf = 3;           // token-tile buffers: compute + two in flight
constexpr float kRescaleGap = 8.f; // log2 units: weights may reach 2^8 before m moves

// LDS byte layout: W and W' (128 rows x 256 B), then the token tiles, each
// U^T (128 rows x 128 B) followed by U'^T (128 rows x 128 B).  A tail unit
// uses the whole LDS as its own stages.
constexpr int kWBytes = kMaxR * kD * 2;
constexpr int kOffW = 0;
constexpr int kOffWp = kWBytes;
constexpr int kHalfTile = kMaxR * kTT * 2;
constexpr int kTileBytes = 2 * kHalfTile;
constexpr int kOffTile = 2 * kWBytes;
constexpr int kLdsBytes = kOffTile + kNBuf * kTileBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
// A tail unit's LDS: stages of one 64-token tile, K (64 rows x 256 B) then V.
constexpr int kTailHalf = kTT * kD * 2;
constexpr int kTailStageBytes = 2 * kTailHalf;
constexpr int kTailStages = kLdsBytes / kTailStageBytes;
static_assert(kTailStages == 5, "the tail loop's waits assume 4 tiles in flight");
static_assert(kRowsPerTile == 128, "the host splits query rows in tiles of 128");

// Swizzles (16-byte chunk index XOR a function of the row):
//  W, tail K : 16 chunks per row, read 16 rows x one chunk per 16 lanes
//  W', tail V: 16 chunks per row, transposing reads of 8 rows x 2 chunks
//  U^T       :  8 chunks per row, transposing reads of 8 rows x 2 chunks
//  U'^T      :  8 chunks per row, row reads of 16 rows x one chunk
__device__ __forceinline__ int swz_w(int r) { return r & 15; }
__device__ __forceinline__ int swz_wp(int r) { return (r & 7) << 1; }
__device__ __forceinline__ int swz_u(int r) { return ((r >> 1) & 3) << 1; }
__device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 7; }


// Operands read from a swizzled K-major LDS array (row = K index, columns =
// M, `cpr` 16-byte chunks per row):
//   K = 32: slot s of lane l <- X[row0 + 4(l/16) + s%4 + 16(s/4)][col0 + l%16]
//   K = 16: slot s of lane l <- X[row0 + 4(l/16) + s][col0 + l%16]
// Lane x addresses the 8 bytes at row row0 + 4(x/16) + (x%16)/4, columns
// col0 + 4(x%4) .. +3 (col0 a multiple of 16); the swizzle of a row is the
// same for that row + 16.
template <int CPR, int (*SWZ)(int)>
__device__ __forceinline__ int tr_addr(int row0, int col0, int lane) {
  const int r = row0 + 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int chunk = (col0 >> 3) + ((lane & 3) >> 1);
  return r * (CPR * 16) + ((chunk ^ SWZ(r)) << 4) + ((lane & 1) << 3);
}
template <int CPR, int (*SWZ)(int)>
__device__ __forceinline__ u32x4_t tr_operand(const char* X, int row0, int col0, int lane) {
  const int a = tr_addr<CPR, SWZ>(row0, col0, lane);
  const u32x2_t lo = tr_read(X + a), hi = tr_read(X + a + 16 * CPR * 16);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}
template <int CPR, int (*SWZ)(int)>
__device__ __forceinline__ u32x2_t tr_operand16(const char* X, int row0, int col0, int lane) {
  return tr_read(X + tr_addr<CPR, SWZ>(row0, col0, lane));
}
// K = 32 operand read along rows of the swizzled U'^T tile (row = M index,
// 8 chunks per row, columns = K): slot s of lane l <-
// X[row0 + l%16][col0 + 4(l/16) + s%4 + 16(s/4)], col0 a multiple of 32.
__device__ __forceinline__ u32x4_t v_operand(const char* X, int row0, int col0, int lane) {
  const int r = row0 + (lane & 15);
  const int c0 = (col0 >> 3) + (lane >> 5), half = ((lane >> 4) & 1) << 3;
  const int s = swz_v(r);
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(X + r * 128 + ((c0 ^ s) << 4) + half);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(X + r * 128 + (((c0 + 2) ^ s) << 4) + half);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}
// A operand from a swizzled row-major 256-byte-row array (W, tail K): slot s
// of lane l <- X[row0 + l%16][kc*32 + 8(l/16) + s].
__device__ __forceinline__ u32x4_t w_operand(const char* X, int row0, int kc, int lane) {
  const int r = row0 + (lane & 15);
  const int chunk = 4 * kc + (lane >> 4);
  return *reinterpret_cast<const u32x4_t*>(X + r * 256 + ((chunk ^ swz_w(r)) << 4));
}

// vmcnt(N) (lgkmcnt(0), expcnt untouched), then a workgroup barrier.  No
// memory fence: loads issued after the awaited ones stay in flight.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A block's factor layout (wave-uniform).
struct BlockInfo {
  const uint16_t* head;   // this KV head's factors
  uint32_t bytes;         // their size
  int T, ld, r, rv, nk, nv, ntiles;
  uint32_t w_off, v_off, wp_off;
};

// Buffer resource of a block's factors.
__device__ __forceinline__ u32x4_t rsrc_of(const BlockInfo& io) { return rsrc_words(io.head, io.bytes); }

// The block table is read through the constant address space: it does not
// change during the kernel, so its (wave-uniform) reads stay scalar loads
// even though the DMA asm counts as a memory clobber.
typedef __attribute__((address_space(4))) const milo_block const_milo_block;

template <int HD>
__device__ __forceinline__ void block_info(BlockInfo& io, const ChunkParams& p, int gblk, int g) {
  const_milo_block* blk = (const_milo_block*)p.blocks + gblk;
  constexpr int hd = HD;
  io.T = max(blk->n_tok, 0);
  io.ld = blk->ld_tok;
  io.r = min(max(blk->rank_k, 0), hd);
  io.rv = min(max(blk->rank_v, 0), hd);
  // 16-rank chunks: scores use at least one (a rank-0 block scores 0
  // against zero-padded factors); values use none for rank' 0
  io.nk = max(1, (io.r + 15) / 16);
  io.nv = (io.rv + 15) / 16;
  io.ntiles = max(1, (io.T + kTT - 1) / kTT);
  io.head = reinterpret_cast<const uint16_t*>(p.pool) + blk->off +
            (int64_t)g * (io.r + io.rv) * (io.ld + hd);
  io.bytes = (uint32_t)((io.r + io.rv) * (io.ld + hd)) * 2;
  io.w_off = (uint32_t)(io.r * io.ld) * 2;
  io.v_off = io.w_off + (uint32_t)(io.r * hd) * 2;
  io.wp_off = io.v_off + (uint32_t)(io.rv * io.ld) * 2;
}

// Token tile starting at t0 into tile buffer `buf` (4 loads per wave): load
// k of wave w moves 8 rows (row block 8k + w of the 32 row blocks: U^T
// 0-15, U'^T 16-31) x 8 chunks, lane l taking row (l/8) of the row block
// and LDS chunk position l%8.  Rows past the rank and chunks past the
// block's padded length load zeros.
__device__ __forceinline__ void issue_tile(const BlockInfo& io, char* buf, int t0, int lane, int wave) {
  const u32x4_t rs = rsrc_of(io);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool is_v = k >= 2;
    const int rb = (k & 1) * 8 + wave;
    const int row = rb * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (is_v ? swz_v(row) : swz_u(row));
    const uint32_t off = (is_v ? io.v_off : 0u) + (uint32_t)(row * io.ld + t0 + chunk * 8) * 2;
    // chunks that start past the block's last token load zeros: row padding
    // beyond it may hold anything (NaN included) and would meet e = 0 in the
    // value MFMA (0 * NaN = NaN); the partial chunk at n_tok is masked later
    const bool ok = row < (is_v ? io.rv : io.r) && t0 + chunk * 8 < io.T;
    dma16(rs, buf + (is_v ? kHalfTile : 0) + rb * 1024, off, ok);
  }
}
// W (wp = false) or W' rows of a block into their LDS region (4 loads per
// wave: row block 8k + w of 32, 4 rows x 16 chunks each).
template <int HD>
__device__ __forceinline__ void issue_w(const BlockInfo& io, char* region, bool wp, int lane, int wave) {
  const u32x4_t rs = rsrc_of(io);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rb = 8 * k + wave;
    const int row = rb * 4 + (lane >> 4);
    const int chunk = (lane & 15) ^ (wp ? swz_wp(row) : swz_w(row));
    // head_dim 64: the upper half of each 128-wide LDS row loads zeros
    const uint32_t off = (wp ? io.wp_off : io.w_off) + (uint32_t)(row * HD + chunk * 8) * 2;
    dma16(rs, region + rb * 1024, off, row < (wp ? io.rv : io.r) && chunk * 8 < HD);
  }
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

template <int HD>
__global__ __launch_bounds__(kThreads) void milo_chunk_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.group;
  char* const ldsW = lds + kOffW;
  char* const ldsWp = lds + kOffWp;
  auto tile_buf = [&](int k) { return lds + kOffTile + (k % kNBuf) * kTileBytes; };

  // workgroup -> (sequence, KV head, range slot, query tile).  The first
  // ceil(groups / 8) * 8 * n_qtiles workgroups are dispatched round-robin
  // over the 8 XCDs: slot k of XCD x runs query tile k % n_qtiles of group
  // (k / n_qtiles) * 8 + x.  A shared-context launch then has tail_units
  // more, each the dense tail of one (sequence i, KV head g) for its one
  // query token; placed last, they take the CUs that finish first.
  const int S = p.n_ranges + p.tail_pieces;
  const int n_groups = p.batch * p.n_kv_heads * S;
  const int n_block_wgs = (n_groups + 7) / 8 * 8 * p.n_qtiles;
  const bool extra = (int)blockIdx.x >= n_block_wgs;
  int i, g, slot, qt, qlen;
  if (extra) {
    const int u = (int)blockIdx.x - n_block_wgs;
    if (u >= p.tail_units) return;
    i = u / (p.n_kv_heads * p.tail_pieces);
    g = (u / p.tail_pieces) % p.n_kv_heads;
    slot = p.n_ranges + u % p.tail_pieces;
    qt = 0;
    qlen = 1;
  } else {
    const int bid = blockIdx.x;
    const int xcd = bid & 7, k8 = bid >> 3;
    const int group = (k8 / p.n_qtiles) * 8 + xcd;
    if (group >= n_groups) return;
    qt = k8 % p.n_qtiles;
    slot = group % S;
    g = (group / S) % p.n_kv_heads;
    i = group / (S * p.n_kv_heads);
    qlen = p.q_len;
  }

  const int MQ = qlen * G;
  const int m_l = qt * kRowsPerTile + wave * kRowsPerWave + (lane & 15);  // this lane's column
  const bool row_ok = m_l < MQ;
  // A wave whose 16 rows all lie past the last query row skips the MFMA and
  // softmax work (it still issues its share of every load and joins every
  // barrier), leaving its SIMD to the other wave.
  const bool wave_live = qt * kRowsPerTile + wave * kRowsPerWave < MQ;
  const int j_l = m_l / G, hl = m_l - j_l * G;

  const bool tail = slot >= p.n_ranges;
  if (tail && p.no_tail && !extra) return;
  int b0 = 0, blk_lo = 0, blk_hi = 0;
  if (!tail) {
    b0 = p.seq_blocks[i];
    const int nb = min(max(p.seq_blocks[i + 1] - b0, 0), p.max_blocks);
    blk_lo = slot * p.blocks_per_range;
    blk_hi = min(nb, blk_lo + p.blocks_per_range);
    if (blk_lo >= blk_hi) return;   // empty range: the merge skips it
  }

  // Q^T operand chunks qv[kk] = q[row m_l][32kk + 8(l/16) .. +8], held for
  // the whole unit.  Lanes past the last row read row 0: their columns are
  // never written out.  Loaded after the unit's first DMA loads and awaited
  // at once (vmcnt(0)): a wait left to the compiler would sit in the block
  // loop and also drain the prefetched tiles at every block.
  u32x4_t qv[kD / 32];
  auto load_q = [&]() {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           (((int64_t)i * qlen + (row_ok ? j_l : 0)) * p.n_q_heads + g * G +
                            (row_ok ? hl : 0)) * HD + 8 * q4;
    // dims past head_dim (64) are zero in every operand
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk)
      qv[kk] = 32 * kk + 8 * q4 < HD ? ld16(qrow + 32 * kk) : u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
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
  // score exceeds it by more than kRescaleGap, rescaling O, Z and l, and
  // returns e = exp2(s_true - m) as two K = 32 bf16 operands.
  auto softmax64 = [&](f32x4_t (&s)[4], float mref, u32x4_t (&eb)[2]) {
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
        for (int zt = 0; zt < kMaxR / 16; ++zt) Z[zt] *= alpha;
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
    // Pipeline over the unit's tiles k = 0, 1, ...: tile k + 2 is issued at
    // step k, after the step's barrier (its buffer was last read at step
    // k - 1).  Every step waits with vmcnt(4): all loads but the newest tile
    // (issued at step k - 1, after any W / W' loads of that step) are done.
    BlockInfo cb, pb;                     // compute block, prefetch block
    block_info<HD>(cb, p, b0 + blk_lo, g);
    pb = cb;
    int pblk = blk_lo, pt = 0;            // next tile to issue: block pblk, tile pt
    int kpre = 0;                         // global index of that tile
    auto advance_pre = [&]() {
      ++kpre;
      if (++pt >= pb.ntiles) {
        pt = 0;
        if (++pblk < blk_hi) {
          block_info<HD>(pb, p, b0 + pblk, g);
              }
      }
    };
    auto issue_next = [&](int ln) -> bool {
      if (pblk >= blk_hi) return false;
      issue_tile(pb, tile_buf(kpre), pt * kTT, ln, wave);
      advance_pre();
      return true;
    };
    // W of block b + 1 goes into ldsW during block b's last tile.  It is
    // taken from that block's own descriptor: the prefetch cursor pb is two
    // tiles ahead and already past b + 1 when b + 1 has a single tile.
    int cur_b = blk_lo;
    auto issue_next_w = [&](int ln) {
      BlockInfo nb;
      block_info<HD>(nb, p, b0 + cur_b + 1, g);
      issue_w<HD>(nb, ldsW, false, ln, wave);
    };
    issue_w<HD>(cb, ldsW, false, lane, wave);
    issue_w<HD>(cb, ldsWp, true, lane, wave);
    issue_next(lane);
    bool newest = issue_next(lane);           // was a tile issued at the previous step?
    load_q();
    int k = 0;                            // global index of the tile computed now

    for (int b = blk_lo; b < blk_hi; ++b) {
      cur_b = b;
      if (b > blk_lo) block_info<HD>(cb, p, b0 + b, g);
      const int T = cb.T, r = cb.r, nv = cb.nv, ntiles = cb.ntiles;
      const bool has_next = b + 1 < blk_hi;
#pragma unroll
      for (int zt = 0; zt < kMaxR / 16; ++zt) Z[zt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // Everything that depends on the number of 16-rank score chunks is
      // compiled per count, so the MFMA chains are straight-line code.
      auto body = [&](auto nk_c) {
        constexpr int NK = decltype(nk_c)::value;
        constexpr int NK2 = NK / 2;           // K = 32 chunks
        constexpr bool REM = (NK & 1) != 0;   // trailing K = 16 chunk
        u32x4_t ph[NK2 > 0 ? NK2 : 1], pl[NK2 > 0 ? NK2 : 1];
        u32x2_t ph16, pl16;
        for (int t = 0; t < ntiles; ++t, ++k) {
          if (newest) wait_barrier<4>(); else wait_barrier<0>();
          const int ln = opaque(lane);
          const char* U = tile_buf(k);
          const char* V = U + kHalfTile;
          const int t0 = t * kTT;
          if (t == 0) {
            if (b > blk_lo) issue_w<HD>(cb, ldsWp, true, ln, wave);   // W' of this block
            // ---- P^T = W Q^T per 16-rank tile, scaled, split into hi/lo operands
            f32x4_t pt[NK];
            if (wave_live) {
#pragma unroll
            for (int rt = 0; rt < NK; ++rt) {
              f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kk = 0; kk < kD / 32; ++kk)
                acc = mfma32(w_operand(ldsW, 16 * rt, kk, ln), qv[kk], acc);
#pragma unroll
              for (int v = 0; v < 4; ++v)
                acc[v] = (16 * rt + 4 * q4 + v < r) ? acc[v] * p.scale_log2 : 0.f;
              pt[rt] = acc;
            }
#pragma unroll
            for (int j = 0; j < NK2; ++j) split_pair(pt[2 * j], pt[2 * j + 1], ph[j], pl[j]);
            if (REM) split_one(pt[NK - 1], ph16, pl16);
            }
            if (ntiles == 1 && has_next) {   // W is read: the next block's may land
              wait_barrier<63>();
              issue_next_w(ln);
            }
          } else if (t == ntiles - 1 && has_next) {
            issue_next_w(ln);   // W of the next block
          }
          newest = issue_next(ln);
          if (t0 + kTT > T && (T & 7)) {
            // U'^T tokens past the block end in the tile's last partial chunk
            // (row padding) are zeroed: they meet e = 0 in the MFMA.
            if (tid < kMaxR) {
              const int c = (T - t0) >> 3, n = (T - t0) & 7;
              u32x4_t* pv = reinterpret_cast<u32x4_t*>(const_cast<char*>(V) + tid * 128 +
                                                       ((c ^ swz_v(tid)) << 4));
              u32x4_t v = *pv;
#pragma unroll
              for (int w = 0; w < 4; ++w)
                v[w] &= (2 * w < n ? 0xffffu : 0u) | (2 * w + 1 < n ? 0xffff0000u : 0u);
              *pv = v;
            }
            wait_barrier<63>();
          }

          if (!wave_live) continue;   // no query rows in this wave
          // ---- S^T = U P^T (hi + lo) for the tile's four 16-token blocks,
          // chunk-outer so that the four chains' reads are in flight
          // together; the chains start from -mref, so scores arrive
          // relative to it.
          const float mref = score_ref();
          const f32x4_t bias = {-mref, -mref, -mref, -mref};
          f32x4_t s[4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) s[tt] = bias;
#pragma unroll
          for (int j = 0; j < NK2; ++j) {
            u32x4_t a[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) a[tt] = tr_operand<8, swz_u>(U, 32 * j, 16 * tt, ln);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              s[tt] = mfma32(a[tt], ph[j], s[tt]);
              s[tt] = mfma32(a[tt], pl[j], s[tt]);
            }
          }
          if (REM) {
            u32x2_t a[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) a[tt] = tr_operand16<8, swz_u>(U, 32 * NK2, 16 * tt, ln);
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
          softmax64(s, mref, eb);
          // ---- Z^T += U'^T E^T, pairs of rank' tiles, four reads in flight
#pragma unroll
          for (int vt = 0; vt < kMaxR / 16; vt += 2) {
            if (vt < nv) {
              u32x4_t a[4];
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                a[c] = v_operand(V, 16 * vt, 32 * c, ln);
                a[2 + c] = v_operand(V, 16 * vt + 16, 32 * c, ln);
              }
#pragma unroll
              for (int c = 0; c < 2; ++c) Z[vt] = mfma32(a[c], eb[c], Z[vt]);
              if (vt + 1 < nv) {
#pragma unroll
                for (int c = 0; c < 2; ++c) Z[vt + 1] = mfma32(a[2 + c], eb[c], Z[vt + 1]);
              }
            }
          }
        }
      };
      switch (cb.nk) {
        case 1: body(IntC<1>{}); break;
        case 2: body(IntC<2>{}); break;
        case 3: body(IntC<3>{}); break;
        case 4: body(IntC<4>{}); break;
        case 5: body(IntC<5>{}); break;
        case 6: body(IntC<6>{}); break;
        case 7: body(IntC<7>{}); break;
        default: body(IntC<8>{}); break;
      }

      // ---- O^T += W'^T Z^T.  W' was issued at this block's first step; a
      // single-tile block waits for it here.  Its rows past rank' are zero,
      // as are Z's.
      if (ntiles == 1) wait_barrier<0>();
      const int ln = opaque(lane);
#pragma unroll
      for (int j = 0; j < kMaxR / 32; ++j) {
        if (!wave_live) break;
        if (2 * j + 1 < nv) {
          u32x4_t zh, zl;
          split_pair(Z[2 * j], Z[2 * j + 1], zh, zl);
#pragma unroll
          for (int dt = 0; dt < kD / 16; ++dt) {
            const u32x4_t a = tr_operand<16, swz_wp>(ldsWp, 32 * j, 16 * dt, ln);
            O[dt] = mfma32(a, zh, O[dt]);
            O[dt] = mfma32(a, zl, O[dt]);
          }
        } else if (2 * j < nv) {
          u32x2_t zh, zl;
          split_one(Z[2 * j], zh, zl);
#pragma unroll
          for (int dt = 0; dt < kD / 16; ++dt) {
            const u32x2_t a = tr_operand16<16, swz_wp>(ldsWp, 32 * j, 16 * dt, ln);
            O[dt] = mfma16(a, zh, O[dt]);
            O[dt] = mfma16(a, zl, O[dt]);
          }
        }
      }
    }
    // no load of this unit is left in flight (the last steps issued none)
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    // ---- dense causal tail: token l is visible to query j iff l <= L - Q + j.
    // 64-token tiles of K and V through kTailStages LDS stages of 32 KB (the
    // unit uses no other LDS), up to kTailStages - 1 tiles in flight.  Every
    // lane issues 4 loads per tile, so tile t is in LDS once at most 4 * n
    // loads are pending, n = tiles issued after it.
    const int cap = p.tail_cap;
    const int L = cap > 0 ? min(max(p.tail_len[i], 0), cap) : 0;   // tail_len may be NULL if cap is 0
    constexpr int hd = HD;
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(p.k_tail) + ((size_t)i * p.n_kv_heads + g) * cap * hd;
    const uint16_t* vtp = reinterpret_cast<const uint16_t*>(p.v_tail) + ((size_t)i * p.n_kv_heads + g) * cap * hd;
    const u32x4_t rk = rsrc_words(kt, (uint32_t)(cap * hd) * 2);
    const u32x4_t rvv = rsrc_words(vtp, (uint32_t)(cap * hd) * 2);
    const int vis = L - qlen + j_l;   // last visible tail token of this row
    // this unit's piece of the tail: tiles toff .. toff + nt - 1
    const int tpp = ((cap + kTT - 1) / kTT + p.tail_pieces - 1) / p.tail_pieces;
    const int toff = (slot - p.n_ranges) * tpp;
    const int nt = max(0, min((L + kTT - 1) / kTT, toff + tpp) - toff);
    auto stage = [&](int t) { return lds + (t % kTailStages) * kTailStageBytes; };
    auto issue_tail = [&](int t) {
      const int ln = opaque(lane);
      char* const sk = stage(t);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int rb = 8 * k + wave;
        const int row = rb * 4 + (ln >> 4);
        const int tok = (toff + t) * kTT + row;
        const int ck = (ln & 15) ^ swz_w(row), cv = (ln & 15) ^ swz_wp(row);
        dma16(rk, sk + rb * 1024, (uint32_t)(tok * hd + ck * 8) * 2, tok < L && ck * 8 < hd);
        dma16(rvv, sk + kTailHalf + rb * 1024, (uint32_t)(tok * hd + cv * 8) * 2, tok < L && cv * 8 < hd);
      }
    };
    for (int t = 0; t < min(nt, kTailStages - 1); ++t) issue_tail(t);
    load_q();   // also waits for this lane's tile loads
    for (int t = 0; t < nt; ++t) {
      // tile t complete in every wave; stage (t + 4) % 5, read at step t - 1, is free
      switch (min(nt - 1, t + kTailStages - 2) - t) {
        case 3: wait_barrier<12>(); break;
        case 2: wait_barrier<8>(); break;
        case 1: wait_barrier<4>(); break;
        default: wait_barrier<0>(); break;
      }
      if (t + kTailStages - 1 < nt) issue_tail(t + kTailStages - 1);
      if (!wave_live) continue;   // no query rows in this wave
      const int ln = opaque(lane);
      char* const sk = stage(t);
      // S^T = K_tail q^T (K = d), scaled, relative to mref, causally masked
      const float mref = score_ref();
      f32x4_t s[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk) acc = mfma32(w_operand(sk, 16 * tt, kk, ln), qv[kk], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = (toff + t) * kTT + 16 * tt + 4 * q4 + v;
          acc[v] = (tok < L && tok <= vis) ? acc[v] * p.scale_log2 - mref : kNegInf;
        }
        s[tt] = acc;
      }
      u32x4_t eb[2];
      softmax64(s, mref, eb);
      // O^T += V_tail^T E^T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < kD / 16; ++dt)
          O[dt] = mfma32(tr_operand<16, swz_wp>(sk + kTailHalf, 32 * c, 16 * dt, ln), eb[c], O[dt]);
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
    const int si = i + m_l / p.part_rows, ml = m_l % p.part_rows;
    const size_t rec = ((size_t)((si * p.n_kv_heads + g) * S + slot)) * p.part_rows + ml;
    float* po = p.part.o + rec * HD;
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt)
      if (16 * dt < HD) *reinterpret_cast<f32x4_t*>(po + 16 * dt + 4 * q4) = O[dt];
    if (q4 == 0) {
      p.part.ml[rec * 2 + 0] = m_run;
      p.part.ml[rec * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_chunk(const ChunkParams& p, int group, hipStream_t s, LaunchEvents ev) {
  const int64_t groups = (int64_t)p.batch * p.n_kv_heads * (p.n_ranges + p.tail_pieces);
  if (groups == 0) return hipSuccess;
  if (group < 1 || group > 16) return hipErrorInvalidValue;
  const int64_t wgs = (p.tail_units + 7) / 8 * 8 + (groups + 7) / 8 * 8 * p.n_qtiles;
  ChunkParams q = p;
  q.group = group;
  auto kernel = p.head_dim == 64 ? milo_chunk_kernel<64> : milo_chunk_kernel<128>;
  if (ev.start && ev.stop)   // timing events stamped by the dispatch itself
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(kThreads), 0, s, ev.start, ev.stop, 0, q);
  else
    hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(kThreads), 0, s, q);
  return hipGetLastError();
}

}  // namespace milo
