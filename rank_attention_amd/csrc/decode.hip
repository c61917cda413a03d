// decode.hip -- gfx950 decode attention over a block-wise low-rank KV cache.
//
// MILO (summary at paperlayer.ai/abs/2609.29913v1) stores each block's keys
// and values as separate low-rank factors, K_b ~= U_b W_b and V_b ~= U'_b W'_b
// ("4.2 Block-wise Low-Rank Compression"), and at inference attends over the
// selected blocks ("4.4 MILO Workflow").  This kernel evaluates that attention
// in the absorbed order, which never forms K_b or V_b:
//     p = scale*log2(e) * W_b q     s = U_b p     e = exp2(s - m)
//     z = e^T U'_b                  o~ = z W'_b
// and leaves per-unit partials (o~, m, l) for the merge kernel.
//
// Work unit = one wave (64 lanes) per (sequence, KV head, block slot), plus
// one dense-tail unit per (sequence, KV head).  The G query heads of the KV
// group share every factor load.  The block's token factors are streamed
// once, rank-major, 16 bytes per lane:
//   - scores: lane owns 16 tokens of a 1024-token tile (two 1 KB wave-wide
//     row segments; a block of at most 512 tokens: 8 tokens per lane of a
//     512-token tile, and 16 rows per load stage instead of 4).  Every four
//     rows of U^T are one K = 4 step of v_mfma_f32_4x4x4bf16_1k: the lane's
//     token is a column of B (two byte permutes of its row loads), p of four
//     heads the rows of A, split into bf16 hi + lo; the lane keeps the
//     scores of its own tokens;
//   - values: the same lane/token ownership; e is packed to bf16 token pairs
//     against rows of U'^T; per-lane partial z of up to 64 (row, head) slots
//     are summed across the wave by one transposing butterfly; the next row
//     group's first rows load during that reduction;
//   - o~ += z W' is applied per row group as soon as the group's z is
//     reduced; the group's W' rows load with its U'^T rows, so no memory
//     round trip is left after the last group.
// The softmax max, sum and rescale factor are wave-uniform and kept in
// scalar registers.
// The U^T and U'^T streams are read once and wave-coalesced, so they are
// loaded non-temporally.  The projection p = W q (bf16 storage) runs on the
// matrix cores with all of the unit's W loads in flight at once (one memory
// round trip).  A unit is one wave, so LDS
// hand-offs between its lanes need no barrier (a barrier would also wait
// for every load in flight).
//
// That is the path of bf16 and fp32 storage.  With 8-bit token factors
// (MILO_BF16_Q8) the same work units run the scores and the value side on
// the matrix cores instead (block_unit_q8 and milo_decode_q8_kernel below):
// the codes are exact fp16 operands, so the vector ALUs are left with the
// softmax and o~ += z W'.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kLdsWords = 2560;   // p (4 KB) | z partials (4 KB) | q of the group (2 KB)
constexpr float kNegInf = -__builtin_huge_valf();

template <int D, int G>
struct Shape {
  // value rows per butterfly group (R * G <= 64 slots); G = 5 takes 11 so
  // that the bf16 unit's value phase fits two waves per SIMD
  static constexpr int R = G == 5 ? 11 : (64 / G < 12) ? 64 / G : 12;
  static constexpr int NG = (D + R - 1) / R;    // butterfly groups for rank <= D
  static constexpr int JPL = D / 64;            // output columns per lane
  static_assert(G >= 1 && G <= 8, "group size");
  static_assert(NG * 64 <= 1024, "z staging fits its LDS region");
};

// ---------------------------------------------------------------------------
// bf16 storage
// ---------------------------------------------------------------------------

// Orders this wave's LDS writes before its later LDS reads for the
// compiler.  A unit is one wave, and the LDS executes one wave's requests
// in order, so no barrier (which would also wait for every load in flight)
// is needed.
__device__ __forceinline__ void wave_lds_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// p = scale*log2(e) * W q for the G heads (fp32) on the matrix cores: P^T
// (16 ranks x 16 heads) per tile of 16 rows of W, K = head_dim in steps of
// 32 (exact bf16 products, fp32 sums).  Lane l loads 8 dims 32s + 8(l/16) .. +7 of W row 16t + l%16
// (clamped to r-1) and of q head l%16 (zero for l%16 >= G); the result
// holds ranks 16t + 4(l/16) + v of head l%16, written to pf[rank*8 + head]
// for heads < G.  Every W load of the unit is issued first (one round
// trip).  Rows >= r of pf are not meaningful.  Requires r >= 1.
template <int D, int G>
__device__ __forceinline__ void mfma_project_q(const uint16_t* W, const uint16_t* qh, int r, float scale_log2,
                                               float* pf, int lane) {
  constexpr int KS = D / 32, MT = D / 16;   // K steps; rank tiles for r <= D
  const int quad = lane >> 4, col = lane & 15;
  const int nt = (r + 15) >> 4;
  u32x4_t qb[KS], wt[MT][KS];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    if (t < nt) {
      const uint16_t* row = W + (size_t)min(16 * t + col, r - 1) * D + 8 * quad;
#pragma unroll
      for (int k = 0; k < KS; ++k) wt[t][k] = ld16(row + 32 * k);
    }
#pragma unroll
  for (int k = 0; k < KS; ++k)
    qb[k] = col < G ? ld16(qh + (size_t)col * D + 32 * k + 8 * quad) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < MT; ++t)
    if (t < nt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) acc = mfma_bf16(wt[t][k], qb[k], acc);
      if (col < G) {
#pragma unroll
        for (int v = 0; v < 4; ++v) pf[(16 * t + 4 * quad + v) * 8 + col] = acc[v] * scale_log2;
      }
    }
}

// U^T rows per prefetch step of the score loop (two steps in flight): 4
// with two 8-token chunks per lane, 16 with one, whose scores take half
// the registers.  Units of blocks of at most 512 tokens are latency-bound
// (few units per wave slot), so fewer, larger round trips shorten them.
template <int CH>
constexpr int rows_per_step() { return CH == 1 ? 16 : 4; }

// U'^T rows of the next value group whose loads are issued during this
// group's reduction: the whole group with one chunk per lane, else as many
// as the two-waves-per-SIMD register budget leaves room for.
template <int G, int CH, int R>
constexpr int value_ring_rows() { return CH == 1 ? R : 0; }

// Loads rows k0 .. k0 + rows_per_step - 1 of U^T (clamped to r-1) at the
// lane's CH chunks.
template <int CH>
__device__ __forceinline__ void load_rows(const uint16_t* Ut, int ld, int k0, int r, const int (&tq)[CH],
                                           u32x4_t (&A)[CH][rows_per_step<CH>()]) {
#pragma unroll
  for (int j = 0; j < rows_per_step<CH>(); ++j) {
    const uint16_t* row = Ut + (size_t)min(k0 + j, r - 1) * ld;
#pragma unroll
    for (int c = 0; c < CH; ++c) A[c][j] = ld16_stream(row + tq[c]);
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

// v_mfma_f32_4x4x4bf16_1k: 16 independent 4x4x4 products, one per group of
// four lanes 4b .. 4b+3.  Lane 4b + j supplies column j of B (K = 4 values)
// and receives column j of D (rows 0..3); lane 4b + v supplies row v of A.
__device__ __forceinline__ f32x4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, const f32x4_t& c) {
  const u32x2v_t a = {a0, a1}, b = {b0, b1};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                 c, 0, 0, 0);
}

// Scores of rows k0 .. k0 + rows_per_step - 1 of U^T on the matrix cores, in
// groups of four rows (K = 4): the lane's token j is column j of B, built
// from its four row loads by two byte permutes, and A holds p of heads
// 4 hg .. 4 hg + 3 (lane 4b + v: head 4 hg + v) at those ranks, split into
// bf16 hi + lo (two products; bf16 U times bf16 p is exact, sums in fp32).
// acc[token][hg] row v = score of head 4 hg + v.  Ranks past r and heads
// past G take p = 0, so the clamped row loads add nothing.
template <int G, int CH>
__device__ __forceinline__ void score_rows_mfma(const u32x4_t (&A)[CH][rows_per_step<CH>()], int k0, int r,
                                                const float* pf, f32x4_t (&acc)[8 * CH][(G + 3) / 4], int lane) {
  constexpr int RPS = rows_per_step<CH>(), HG = (G + 3) / 4;
  const int hv = lane & 3;
#pragma unroll
  for (int kq = 0; kq < RPS / 4; ++kq) {
    const int kb = k0 + 4 * kq;
    if (kb < r) {
      uint32_t ahi[HG][2], alo[HG][2];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const int h = 4 * hg + hv;
        float x[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) x[kk] = (kb + kk < r && h < G) ? pf[(kb + kk) * 8 + h] : 0.f;
        ahi[hg][0] = pack_bf16(x[0], x[1]);
        ahi[hg][1] = pack_bf16(x[2], x[3]);
        alo[hg][0] = pack_bf16(x[0] - bf_lo(ahi[hg][0]), x[1] - bf_hi(ahi[hg][0]));
        alo[hg][1] = pack_bf16(x[2] - bf_lo(ahi[hg][1]), x[3] - bf_hi(ahi[hg][1]));
      }
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t b0 = __builtin_amdgcn_perm(A[c][4 * kq + 1][j >> 1], A[c][4 * kq][j >> 1], sel);
          const uint32_t b1 = __builtin_amdgcn_perm(A[c][4 * kq + 3][j >> 1], A[c][4 * kq + 2][j >> 1], sel);
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            acc[8 * c + j][hg] = mfma4(ahi[hg][0], ahi[hg][1], b0, b1, acc[8 * c + j][hg]);
            acc[8 * c + j][hg] = mfma4(alo[hg][0], alo[hg][1], b0, b1, acc[8 * c + j][hg]);
          }
        }
    }
  }
}


// One tile of 512 CH tokens at a time (lane l holds tokens t0 + 512 c + 8 l
// .. +7 of chunk c): scores, online softmax, then per group of R rows of
// U'^T the group's z = e^T U' and at once o~ += z W' for those rows (W'
// rows load with the group), so no pass over W' is left at the end.  o~ is
// rescaled with the softmax like l.  Blocks of at most 512 tokens take CH =
// 1, so no lane carries a chunk that lies wholly past the block.
template <int D, int G, bool RAGGED, int CH>
__device__ __forceinline__ void bf16_tiles(const uint16_t* Ut, const uint16_t* Upt,
                                           const uint16_t* Wp, int ld, int T, int r, int rv,
                                           const float* pf, float (&m_run)[G], float (&l_run)[G],
                                           float (&o)[G][D / 64], float* zs, int lane) {
  using S = Shape<D, G>;
  constexpr int R = S::R, JPL = S::JPL, NE = 8 * CH, RING = value_ring_rows<G, CH, R>();
  for (int t0 = 0; t0 < T; t0 += 512 * CH) {
    int tc[CH], tq[CH];
    bool ok[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      tc[c] = t0 + 512 * c + lane * 8;
      ok[c] = tc[c] < T;
      // A lane whose chunk lies past the block end reads the tile's first
      // chunk instead (always in bounds) and its tokens are masked below.
      tq[c] = ok[c] ? tc[c] : t0;
    }

    // ---- scores s[c*8+e][h] for token tc_c + e: bf16 U against p split
    // into bf16 hi + lo on the matrix cores (bf16 rounding of p alone would
    // cost ~1% on sharp softmax)
    constexpr int HG = (G + 3) / 4;
    f32x4_t acc[NE][HG];
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) acc[e][hg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (r > 0) {
      constexpr int kRowsPerStep = rows_per_step<CH>();
      u32x4_t A0[CH][kRowsPerStep], A1[CH][kRowsPerStep];
      load_rows<CH>(Ut, ld, 0, r, tq, A0);
      for (int k0 = 0; k0 < r; k0 += 2 * kRowsPerStep) {
        if (k0 + kRowsPerStep < r) load_rows<CH>(Ut, ld, k0 + kRowsPerStep, r, tq, A1);
        score_rows_mfma<G, CH>(A0, k0, r, pf, acc, lane);
        if (k0 + 2 * kRowsPerStep < r) load_rows<CH>(Ut, ld, k0 + 2 * kRowsPerStep, r, tq, A0);
        if (k0 + kRowsPerStep < r) score_rows_mfma<G, CH>(A1, k0 + kRowsPerStep, r, pf, acc, lane);
      }
    }
    float s[NE][G];
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int h = 0; h < G; ++h) s[e][h] = acc[e][h >> 2][h & 3];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int tok = tc[e >> 3] + (e & 7);
      if (tok >= T) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[e][h] = kNegInf;
      }
    }

    // ---- online softmax statistics; e packed to bf16 token pairs
    uint32_t e2[CH][4][G];
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int e = 1; e < NE; ++e) mx = fmaxf(mx, s[e][h]);
      mx = wave_max(mx);
      // m, l and alpha are the same in every lane: kept in scalar registers
      const float mn = uniform_f32(fmaxf(m_run[h], mx));
      alpha[h] = uniform_f32(fast_exp2(m_run[h] - mn));
      float sum = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float x0 = fast_exp2(s[c * 8 + 2 * w][h] - mn);
          const float x1 = fast_exp2(s[c * 8 + 2 * w + 1][h] - mn);
          sum += x0 + x1;
          e2[c][w][h] = pack_bf16(x0, x1);
        }
      l_run[h] = uniform_f32(l_run[h] * alpha[h] + wave_sum(sum));
      m_run[h] = mn;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int jj = 0; jj < JPL; ++jj) o[h][jj] *= alpha[h];

    // ---- z = e^T U'  (value factor), reduced per group of R rows, then
    // o~ += z W' for the group.  Rows past rv are loaded clamped to rv-1 and
    // land in slots that are never read.
    // Masks zero the U' elements of tokens past the block end (padding may
    // hold NaN); a lane with no valid token has e = 0 and a finite chunk.
    u32x4_t mask[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      mask[c] = u32x4_t{~0u, ~0u, ~0u, ~0u};
      if (RAGGED) {
        const int n = ok[c] ? T - tc[c] : 0;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          mask[c][w] = (2 * w < n ? 0xffffu : 0u) | (2 * w + 1 < n ? 0xffff0000u : 0u);
      }
    }
    // The first RING rows of a group form a ring: once row rho's products
    // are taken, its registers receive row rho of the next group, so those
    // loads are in flight during this group's reduction and W' update; the
    // group's other rows load at its start.
    u32x4_t U[CH][R];
    uint32_t wr[R];   // the lane's JPL columns of the group's W' rows
    if (rv > 0) {
#pragma unroll
      for (int rho = 0; rho < RING; ++rho) {
        const uint16_t* row = Upt + (size_t)min(rho, rv - 1) * ld;
#pragma unroll
        for (int c = 0; c < CH; ++c) U[c][rho] = ld16_stream(row + tq[c]);
      }
    }
    // group gi; when refill is true the ring takes the next group's rows
    // (every group but the last, so no row is loaded twice)
    auto group = [&](int gi, auto refill) {
#pragma unroll
      for (int rho = RING; rho < R; ++rho) {
        const uint16_t* row = Upt + (size_t)min(gi * R + rho, rv - 1) * ld;
#pragma unroll
        for (int c = 0; c < CH; ++c) U[c][rho] = ld16_stream(row + tq[c]);
      }
#pragma unroll
      for (int rho = 0; rho < R; ++rho) {
        const uint16_t* wrow = Wp + (size_t)min(gi * R + rho, rv - 1) * D;
        wr[rho] = (JPL == 2) ? *reinterpret_cast<const uint32_t*>(wrow + 2 * lane)
                             : (uint32_t)wrow[lane] << 16;
      }
      float acc[64];
#pragma unroll
      for (int x = 0; x < 64; ++x) acc[x] = 0.f;
#pragma unroll
      for (int rho = 0; rho < R; ++rho) {
        u32x4_t u[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          u[c] = U[c][rho];
          if (RAGGED) u[c] &= mask[c];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[rho * G + h] = dot2bf(u[c][w], e2[c][w][h], acc[rho * G + h]);
        if constexpr (decltype(refill)::value) if (rho < RING) {
          const uint16_t* row = Upt + (size_t)min((gi + 1) * R + rho, rv - 1) * ld;
#pragma unroll
          for (int c = 0; c < CH; ++c) U[c][rho] = ld16_stream(row + tq[c]);
        }
      }
      // lane l ends with z of slot l = (row rho, head h); staged in LDS as
      // zs[rho*8 + h] and read back as broadcasts
      const float zg = reduce_transpose64(acc, lane);
      if (lane < R * G) zs[(lane / G) * 8 + lane % G] = zg;
      wave_lds_fence();
#pragma unroll
      for (int rho = 0; rho < R; ++rho) {
        if (gi * R + rho < rv) {
          const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(zs + rho * 8);
          const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(zs + rho * 8 + 4);
          const float zz[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
          const float wv[2] = {bf_lo(wr[rho]), bf_hi(wr[rho])};
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int jj = 0; jj < JPL; ++jj) o[h][jj] = fmaf(zz[h], wv[JPL == 2 ? jj : 1], o[h][jj]);
        }
      }
      wave_lds_fence();
    };
    int gi = 0;
#pragma unroll 1
    for (; (gi + 1) * R < rv; ++gi) group(gi, std::true_type{});
    if (gi * R < rv) group(gi, std::false_type{});
  }
}

template <int D, int G>
__device__ __forceinline__ void block_unit_bf16(const DecodeParams& p, int i, int g, int unit,
                                                const milo_block& blk, uint32_t* lds) {
  using S = Shape<D, G>;
  constexpr int JPL = S::JPL;
  const int lane = threadIdx.x;
  const int T = max(blk.n_tok, 0);
  const int ld = blk.ld_tok;
  const int r = min(max(blk.rank_k, 0), D), rv = min(max(blk.rank_v, 0), D);
  const uint16_t* Ut = reinterpret_cast<const uint16_t*>(p.pool) + blk.off +
                       (int64_t)g * (r + rv) * (ld + D);
  const uint16_t* W = Ut + (size_t)r * ld;
  const uint16_t* Upt = W + (size_t)r * D;
  const uint16_t* Wp = Upt + (size_t)rv * ld;
  const uint16_t* qh = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)i * p.n_q_heads + g * G) * D;

  float* pf = reinterpret_cast<float*>(lds);
  if (r > 0) mfma_project_q<D, G>(W, qh, r, p.scale_log2, pf, lane);
  // z of one row group, staged for broadcast reads: zs[rho*8 + h]
  float* zs = reinterpret_cast<float*>(lds + 1024);

  float m_run[G], l_run[G], o[G][JPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) o[h][jj] = 0.f;
  }
  wave_lds_fence();

  if (T <= 512) {
    if (T & 7)
      bf16_tiles<D, G, true, 1>(Ut, Upt, Wp, ld, T, r, rv, pf, m_run, l_run, o, zs, lane);
    else
      bf16_tiles<D, G, false, 1>(Ut, Upt, Wp, ld, T, r, rv, pf, m_run, l_run, o, zs, lane);
  } else {
    if (T & 7)
      bf16_tiles<D, G, true, 2>(Ut, Upt, Wp, ld, T, r, rv, pf, m_run, l_run, o, zs, lane);
    else
      bf16_tiles<D, G, false, 2>(Ut, Upt, Wp, ld, T, r, rv, pf, m_run, l_run, o, zs, lane);
  }

  float* po = p.part.o + (size_t)unit * G * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) po[h * D + lane * JPL + jj] = o[h][jj];
#pragma unroll
  for (int h = 0; h < G; ++h)
    if (lane == h) {
      p.part.ml[((size_t)unit * G + h) * 2 + 0] = m_run[h];
      p.part.ml[((size_t)unit * G + h) * 2 + 1] = l_run[h];
    }
}

// ---------------------------------------------------------------------------
// 8-bit token factors (MILO_BF16_Q8), on the matrix cores.  Row k of U^T /
// U'^T holds codes c with x = a_k c + b_k; the keys' codes are stored token-
// major ([n_tok][rank_k rounded up to 16]), the values' rank-major in tiles
// of 64 tokens ([n_tok / 64][rank_v][64]).  Folded
// into the absorbed order:
//   s_t = sum_k p_k x_kt  = sum_k (p_k a_k) c_kt + C,   C = sum_k p_k b_k
//   z_k = sum_t e_t x'_kt = a'_k sum_t e_t c'_kt + b'_k E,   E = sum_t e_t
// A byte permute with the constant 0x64 turns four codes into two fp16 pairs
// 1024 + c (exact: the fp16 spacing is 1 on [1024, 2048)), so both sums run
// on v_mfma_f32_16x16x32_f16:
//   scores  S^T (16 tokens x 16 heads) = codes (tokens x ranks) . p'
//           (ranks x heads) with the key codes centred (one packed fp16 add
//           of -1152 gives c - 128, exact) and p' = p a split into fp16
//           hi + lo after scaling by a power of two sc (about 22 mantissa
//           bits); the accumulator starts at sc (C + 128 sum_k p'_k);
//   values  Z^T (16 ranks x 16 heads) = codes' (ranks x tokens) . e (tokens
//           x heads), e rounded to fp16 and the codes left at 1024 + c
//           (all terms positive); l sums those fp16 values, and
//           z = a' (Z - 1024 l) + b' l at the end.
// Heads are the N dimension (G <= 8 of 16 columns used).  A 16x16 result
// holds, in lane l, column l%16 and rows 4(l/16) + v.  Score tile m of a
// 64-token chunk gives row 4j + v token 16j + 4m + v, so after the four
// tiles lane l holds 16 consecutive tokens 16(l/16) .. +15 of head l%16:
// exactly the value MFMA's B operand (K slot 8(l/16) + i = token 16(l/16) +
// i, and + 8 in the second MFMA), against one 16-byte load of a U'^T row.
// A key row's 16-byte load (ranks 16(l/16) .. +15, + 64 for the second
// pair) feeds two K = 32 steps; p' is laid out in that rank order.
// Softmax: the running max m moves only when a chunk's scores exceed it by
// more than 8 (log2 units), so weights stay <= 256, well inside fp16; Z and
// l are rescaled only then.
// ---------------------------------------------------------------------------

constexpr uint32_t kF16Ones = 0x3C003C00u;   // fp16 pair (1, 1)
constexpr uint32_t kF16Magic = 0x64646464u;  // high byte of fp16 1024 + c, c < 256
constexpr int kQ8Chunk = 64;                 // tokens per chunk
constexpr float kQ8Gap = 8.f;                // log2 units the running max may lag

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// fp16 pairs (1024 + c0, 1024 + c1) and (1024 + c2, 1024 + c3) of four codes
__device__ __forceinline__ uint32_t q8_pair_lo(uint32_t c) { return __builtin_amdgcn_perm(kF16Magic, c, 0x04010400u); }
__device__ __forceinline__ uint32_t q8_pair_hi(uint32_t c) { return __builtin_amdgcn_perm(kF16Magic, c, 0x04030402u); }

// The K = 32 operand (8 fp16 of 1024 + c) of codes in words w, w + 1.
__device__ __forceinline__ u32x4_t q8_operand(const u32x4_t& v, int w) {
  u32x4_t a;
  a[0] = q8_pair_lo(v[w]);
  a[1] = q8_pair_hi(v[w]);
  a[2] = q8_pair_lo(v[w + 1]);
  a[3] = q8_pair_hi(v[w + 1]);
  return a;
}

// A code pair centred: (c0 - 128, c1 - 128) = (1024 + c) - 1152, exact in fp16.
// (Each word is centred as it is made: an element-wise loop over the vector
// with the same arithmetic is miscompiled by the toolchain in use.)
__device__ __forceinline__ uint32_t q8_centre(uint32_t pair) {
  const f16x2_t k = {(_Float16)-1152.f, (_Float16)-1152.f};
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, pair) + k);
}

// The K = 32 operand of codes in words w, w + 1, centred.
__device__ __forceinline__ u32x4_t q8_operand_centred(const u32x4_t& v, int w) {
  u32x4_t a;
  a[0] = q8_centre(q8_pair_lo(v[w]));
  a[1] = q8_centre(q8_pair_hi(v[w]));
  a[2] = q8_centre(q8_pair_lo(v[w + 1]));
  a[3] = q8_centre(q8_pair_hi(v[w + 1]));
  return a;
}

__device__ __forceinline__ f32x4_t mfma_f16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                c, 0, 0, 0);
}

// Combine the four lanes l%16 + 16j (j = 0..3) that share a column.
__device__ __forceinline__ float col_max(float v) {
  float a = v, b = v;
  swap16(a, b);
  v = fmaxf(a, b);
  a = v; b = v;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float col_sum(float v) {
  float a = v, b = v;
  swap16(a, b);
  v = a + b;
  a = v; b = v;
  swap32(a, b);
  return a + b;
}

// Registers of the code loads in flight: 16 loads of 16 bytes per lane.  A
// chunk of 64 tokens takes 4 NP key loads (four score tiles, NP pairs of 64
// ranks) at R[KB + NP m + pr] and NTV value loads (tiles of 16 ranks) at
// R[VB + kt].  Units with rank_k, rank_v <= 64 keep two chunks in R, larger
// ones one.
constexpr int kQ8Regs = 16;
typedef u32x4_t Q8Regs[kQ8Regs];

// Geometry of one unit's 8-bit factors (KV head g of one block).
struct Q8Unit {
  const uint8_t* Uk;   // key codes, token-major [T][rk16]
  const uint8_t* Uv;   // value codes, rank-major in 64-token tiles [ld / 64][rv][64]
  int T, ld, r, rv, rk16, npairs, ntv, quad, col;
};

// Code loads of one chunk.  Every address is clamped into the unit's own
// rows (rank offsets to rk16 - 16, tokens to T - 1, value rows to rv - 1),
// so with rank_k, rank_v >= 1 every load is valid and ALL may be issued:
// unguarded (ALL = true), the loop's load counts are static and each wait
// covers only the loads it needs.  The loads are cached (not non-temporal):
// a chunk's key rows are read by its four score tiles in turn.
template <int NP, int KB, bool ALL>
__device__ __forceinline__ void q8_load_keys(Q8Regs& R, const Q8Unit& u, int t0) {
  // key row of score row `col` in tile m: token t0 + 16(col/4) + 4m + col%4
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int tk = min(t0 + 16 * (u.col >> 2) + 4 * m + (u.col & 3), u.T - 1);
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
      if (ALL || pr < u.npairs)
        R[KB + NP * m + pr] = ld16(u.Uk + (size_t)tk * u.rk16 + min(64 * pr + 16 * u.quad, u.rk16 - 16));
  }
}

template <int NTV, int VB, bool ALL>
__device__ __forceinline__ void q8_load_values(Q8Regs& R, const Q8Unit& u, int t0) {
  // tokens t0 + 16 quad .. + 15 of rank row 16 kt + col: the value codes are
  // stored in 64-token tiles [ld / 64][rv][64], so one load instruction
  // reads 16 rows x 64 contiguous bytes
  const uint8_t* tile = u.Uv + (size_t)t0 * u.rv + 16 * u.quad;
#pragma unroll
  for (int kt = 0; kt < NTV; ++kt)
    if (ALL || kt < u.ntv) R[VB + kt] = ld16(tile + (size_t)min(16 * kt + u.col, u.rv - 1) * 64);
}

// Scores of one chunk (consumes its key loads): S[m][v] for token t0 + 16 quad + 4m + v.
template <int NP, int KB>
__device__ __forceinline__ void q8_scores(const Q8Regs& R, const Q8Unit& u, const u32x4_t (&Bh)[NP][2],
                                          const u32x4_t (&Bl)[NP][2], float s0, f32x4_t (&S)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    S[m] = f32x4_t{s0, s0, s0, s0};
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
      if (pr < u.npairs) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4_t a = q8_operand_centred(R[KB + NP * m + pr], 2 * j);
          S[m] = mfma_f16(a, Bh[pr][j], S[m]);
          S[m] = mfma_f16(a, Bl[pr][j], S[m]);
        }
      }
  }
}

// Online softmax of one chunk's scores and Z^T += codes' . e (consumes its value loads).
template <int NTV, int VB>
__device__ __forceinline__ void q8_values(const Q8Regs& R, const Q8Unit& u, const f32x4_t (&S)[4], int t0,
                                          float inv_sc, float& m_run, float& l_run, f32x4_t (&Z)[NTV]) {
  float x[4][4], cmax = kNegInf;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = t0 + 16 * u.quad + 4 * m + v;
      x[m][v] = tok < u.T ? S[m][v] * inv_sc : kNegInf;
      cmax = fmaxf(cmax, x[m][v]);
    }
  cmax = col_max(cmax);
  const bool up = cmax > m_run + kQ8Gap;
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    const float alpha = up ? fast_exp2(m_run - cmax) : 1.f;
    m_run = up ? cmax : m_run;
    l_run *= alpha;
#pragma unroll
    for (int kt = 0; kt < NTV; ++kt)
      if (kt < u.ntv) Z[kt] *= alpha;
  }
  // e = exp2(s - m) as fp16 pairs in token order 16 quad + 0 .. 15
  u32x4_t E0, E1;
  float lp = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t e2 = pack_f16(fast_exp2(x[m][2 * w] - m_run), fast_exp2(x[m][2 * w + 1] - m_run));
      lp = dot2h(e2, kF16Ones, lp);
      if (m < 2) E0[2 * m + w] = e2; else E1[2 * (m - 2) + w] = e2;
    }
  l_run += lp;
#pragma unroll
  for (int kt = 0; kt < NTV; ++kt)
    if (kt < u.ntv) {
      Z[kt] = mfma_f16(q8_operand(R[VB + kt], 0), E0, Z[kt]);
      Z[kt] = mfma_f16(q8_operand(R[VB + kt], 2), E1, Z[kt]);
    }
}

// Loads of chunk c into buffer d of the layout (NP, NTV, DEPTH).
template <int NP, int NTV, int DEPTH, int d, bool ALL>
__device__ __forceinline__ void q8_load_chunk(Q8Regs& R, const Q8Unit& u, int c) {
  constexpr int per = kQ8Regs / DEPTH;
  if (ALL || u.npairs > 0) q8_load_keys<NP, per * d, ALL>(R, u, c * kQ8Chunk);
  if (ALL || u.ntv > 0) q8_load_values<NTV, per * d + 4 * NP, ALL>(R, u, c * kQ8Chunk);
}

// Chunk c from buffer d; PF: issue the loads of chunk c + DEPTH into the
// buffer as it is consumed (keys after the scores, values after the values).
template <int NP, int NTV, int DEPTH, int d, bool ALL>
__device__ __forceinline__ void q8_chunk_step(Q8Regs& R, const Q8Unit& u, int c, bool pf,
                                              const u32x4_t (&Bh)[NP][2], const u32x4_t (&Bl)[NP][2], float s0,
                                              float inv_sc, float& m_run, float& l_run, f32x4_t (&Z)[NTV]) {
  constexpr int per = kQ8Regs / DEPTH;
  static_assert(4 * NP + NTV <= per, "a chunk's loads fit its buffer");
  f32x4_t S[4];
  q8_scores<NP, per * d>(R, u, Bh, Bl, s0, S);
  if (pf && (ALL || u.npairs > 0)) q8_load_keys<NP, per * d, ALL>(R, u, (c + DEPTH) * kQ8Chunk);
  q8_values<NTV, per * d + 4 * NP>(R, u, S, c * kQ8Chunk, inv_sc, m_run, l_run, Z);
  if (pf && (ALL || u.ntv > 0)) q8_load_values<NTV, per * d + 4 * NP, ALL>(R, u, (c + DEPTH) * kQ8Chunk);
}

// The chunk loop: DEPTH chunks in flight, the loads of chunk c + DEPTH going
// out as chunk c consumes its own (the first DEPTH come from q8_preload).
// With rank_k, rank_v >= 1 and at least 2 DEPTH chunks the steady-state
// loop issues every load unguarded (static counts); the last DEPTH chunks,
// and units with an empty factor, take the guarded steps.
// The steady-state loop runs when every load is valid and at least 2 DEPTH chunks exist.
template <int DEPTH>
__device__ __forceinline__ bool q8_steady(const Q8Unit& u) {
  return u.npairs > 0 && u.ntv > 0 && (u.T + kQ8Chunk - 1) / kQ8Chunk >= 2 * DEPTH;
}

// Loads of the first DEPTH chunks (unguarded in the steady case).
template <int NP, int NTV, int DEPTH>
__device__ __forceinline__ void q8_preload(Q8Regs& R, const Q8Unit& u) {
  const int nch = (u.T + kQ8Chunk - 1) / kQ8Chunk;
  if (q8_steady<DEPTH>(u)) {
    q8_load_chunk<NP, NTV, DEPTH, 0, true>(R, u, 0);
    if (DEPTH > 1) q8_load_chunk<NP, NTV, DEPTH, DEPTH - 1, true>(R, u, 1);
  } else {
    if (nch > 0) q8_load_chunk<NP, NTV, DEPTH, 0, false>(R, u, 0);
    if (DEPTH > 1 && nch > 1) q8_load_chunk<NP, NTV, DEPTH, DEPTH - 1, false>(R, u, 1);
  }
}

template <int NP, int NTV, int DEPTH>
__device__ __forceinline__ void q8_chunks(Q8Regs& R, const Q8Unit& u, const u32x4_t (&Bh)[NP][2],
                                          const u32x4_t (&Bl)[NP][2], float s0, float inv_sc, float& m_run,
                                          float& l_run, f32x4_t (&Z)[NTV]) {
  const int nch = (u.T + kQ8Chunk - 1) / kQ8Chunk;
  int c0 = 0;
  if (q8_steady<DEPTH>(u)) {
    for (; c0 + 2 * DEPTH <= nch; c0 += DEPTH) {
      q8_chunk_step<NP, NTV, DEPTH, 0, true>(R, u, c0, true, Bh, Bl, s0, inv_sc, m_run, l_run, Z);
      if (DEPTH > 1)
        q8_chunk_step<NP, NTV, DEPTH, DEPTH - 1, true>(R, u, c0 + 1, true, Bh, Bl, s0, inv_sc, m_run, l_run, Z);
    }
  }
  // the remaining chunks c0 .. nch-1 (fewer than 2 DEPTH); chunks c0 ..
  // c0 + DEPTH - 1 are loaded
  for (; c0 < nch; c0 += DEPTH) {
    q8_chunk_step<NP, NTV, DEPTH, 0, false>(R, u, c0, c0 + DEPTH < nch, Bh, Bl, s0, inv_sc, m_run, l_run, Z);
    if (DEPTH > 1 && c0 + 1 < nch)
      q8_chunk_step<NP, NTV, DEPTH, DEPTH - 1, false>(R, u, c0 + 1, c0 + 1 + DEPTH < nch, Bh, Bl, s0, inv_sc,
                                                      m_run, l_run, Z);
  }
}

// p' = p a (fp32) into the fp16 hi/lo B operands of the rank pairs < NP,
// in the rank order of the key loads; returns this lane's sum of them.
template <int NP, int G>
__device__ __forceinline__ float q8_b_operands(const float* pf, int r, float sc, int quad, int col,
                                               u32x4_t (&Bh)[NP][2], u32x4_t (&Bl)[NP][2]) {
  float psum = 0.f;
#pragma unroll
  for (int pr = 0; pr < NP; ++pr)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float hv[2], lv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int k = 64 * pr + 16 * quad + 8 * j + 2 * w + e;
          const float v = (col < G && k < r) ? pf[k * 8 + col] * sc : 0.f;
          const _Float16 hi = (_Float16)v;
          const _Float16 lo = (_Float16)(v - (float)hi);
          hv[e] = (float)hi;
          lv[e] = (float)lo;
          psum += hv[e] + lv[e];
        }
        Bh[pr][j][w] = pack_f16(hv[0], hv[1]);
        Bl[pr][j][w] = pack_f16(lv[0], lv[1]);
      }
  return psum;
}

// Z (per lane: ranks 16 kt + 4 quad + v, head col) to z = a' (Z - 1024 l) + b' l
// staged as zs[k][h]; (a', b') of every value row are in LDS at abv.
template <int NTV, int G>
__device__ __forceinline__ void q8_stage_z(const f32x4_t (&Z)[NTV], const Q8Unit& u, const float* abv, float l_tot,
                                           float* zs) {
#pragma unroll
  for (int kt = 0; kt < NTV; ++kt)
    if (kt < u.ntv) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int k = 16 * kt + 4 * u.quad + v;
        if (k < u.rv && u.col < G) {
          const f32x2_t ab = *reinterpret_cast<const f32x2_t*>(abv + 2 * k);
          zs[k * 8 + u.col] = fmaf(ab[0], Z[kt][v] - 1024.f * l_tot, ab[1] * l_tot);
        }
      }
    }
}

// Everything between the projection and o~ = z W' for one rank class: the
// B operands, the chunk loop, and z staged in LDS.  Returns m and l (summed
// over the four lanes of each head).
template <int NP, int NTV, int DEPTH, int G>
__device__ __forceinline__ void q8_body(const Q8Unit& u, const float* pf, const float* abv, float* zs, float Cl,
                                        float sc, float inv_sc, float& m_run, float& l_run) {
  Q8Regs R;
  q8_preload<NP, NTV, DEPTH>(R, u);
  u32x4_t Bh[NP][2], Bl[NP][2];
  const float psum = q8_b_operands<NP, G>(pf, u.r, sc, u.quad, u.col, Bh, Bl);
  // the centred codes add -128 sum p' sc to sc * (s - C): start the sum at sc C + that
  const float s0 = fmaf(Cl, sc, 128.f * col_sum(psum));
  f32x4_t Z[NTV];
#pragma unroll
  for (int kt = 0; kt < NTV; ++kt) Z[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  q8_chunks<NP, NTV, DEPTH>(R, u, Bh, Bl, s0, inv_sc, m_run, l_run, Z);
  l_run = col_sum(l_run);
  q8_stage_z<NTV, G>(Z, u, abv, l_run, zs);
}

// o~ = z W' for the G heads of a unit whose z (ranks x 8 heads) is staged in
// LDS at zs, W' rows in groups of 32 (the next group loading while the
// current one is applied); writes the unit's partials (o~, m, l).
template <int D, int G>
__device__ __forceinline__ void store_zwp(const DecodeParams& p, int unit, const uint16_t* Wp, int rv,
                                          const float* zs, float m_run, float l_run, int lane) {
  // o~ = z W' on v_mfma_f32_4x4x4bf16_1k, four W' rows per K step: the
  // lane's output column (dim lane * JPL + jj) is a column of B, packed from
  // its row loads by two byte permutes; row v of A (lane 4b + v) holds z of
  // head 4 hg + v at those rows, split into bf16 hi + lo.  Rows past rank'
  // and heads past G take z = 0 (their W' loads are clamped copies).
  constexpr int JPL = D / 64, HG = (G + 3) / 4;
  const int hv = lane & 3;
  f32x4_t oa[JPL][HG];
#pragma unroll
  for (int jj = 0; jj < JPL; ++jj)
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) oa[jj][hg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int kWRows = 32;
  auto load_w = [&](int k0, uint32_t (&wr)[kWRows]) {
#pragma unroll
    for (int j = 0; j < kWRows; ++j) {
      const uint16_t* wrow = Wp + (size_t)min(k0 + j, rv - 1) * D;
      wr[j] = (JPL == 2) ? *reinterpret_cast<const uint32_t*>(wrow + 2 * lane) : (uint32_t)wrow[lane] << 16;
    }
  };
  uint32_t wa[kWRows], wb[kWRows];
  auto apply_w = [&](int k0, const uint32_t (&wr)[kWRows]) {
#pragma unroll
    for (int j = 0; j < kWRows; j += 4) {
      if (k0 + j < rv) {
        uint32_t ahi[HG][2], alo[HG][2];
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const int h = 4 * hg + hv;
          float x[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) x[kk] = (k0 + j + kk < rv && h < G) ? zs[(k0 + j + kk) * 8 + h] : 0.f;
          ahi[hg][0] = pack_bf16(x[0], x[1]);
          ahi[hg][1] = pack_bf16(x[2], x[3]);
          alo[hg][0] = pack_bf16(x[0] - bf_lo(ahi[hg][0]), x[1] - bf_hi(ahi[hg][0]));
          alo[hg][1] = pack_bf16(x[2] - bf_lo(ahi[hg][1]), x[3] - bf_hi(ahi[hg][1]));
        }
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) {
          // W'[row][dim] sits in the low half of wr for the first of two
          // dims, in the high half for the second (and for JPL = 1)
          const uint32_t sel = (JPL == 2 && jj == 0) ? 0x05040100u : 0x07060302u;
          const uint32_t b0 = __builtin_amdgcn_perm(wr[j + 1], wr[j], sel);
          const uint32_t b1 = __builtin_amdgcn_perm(wr[j + 3], wr[j + 2], sel);
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            oa[jj][hg] = mfma4(ahi[hg][0], ahi[hg][1], b0, b1, oa[jj][hg]);
            oa[jj][hg] = mfma4(alo[hg][0], alo[hg][1], b0, b1, oa[jj][hg]);
          }
        }
      }
    }
  };
  if (rv > 0) load_w(0, wa);
  for (int k0 = 0; k0 < rv; k0 += 2 * kWRows) {
    if (k0 + kWRows < rv) load_w(k0 + kWRows, wb);
    apply_w(k0, wa);
    if (k0 + 2 * kWRows < rv) load_w(k0 + 2 * kWRows, wa);
    if (k0 + kWRows < rv) apply_w(k0 + kWRows, wb);
  }

  float* po = p.part.o + (size_t)unit * G * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) po[h * D + lane * JPL + jj] = oa[jj][h >> 2][h & 3];
  if (lane < G) {
    p.part.ml[((size_t)unit * G + lane) * 2 + 0] = m_run;
    p.part.ml[((size_t)unit * G + lane) * 2 + 1] = l_run;
  }
}

template <int D, int G>
__device__ __forceinline__ void block_unit_q8(const DecodeParams& p, int i, int g, int unit,
                                              const milo_block& blk, uint32_t* lds) {
  const int lane = threadIdx.x;
  Q8Unit u;
  u.quad = lane >> 4;
  u.col = lane & 15;
  u.T = max(blk.n_tok, 0);
  u.ld = blk.ld_tok;
  u.r = min(max(blk.rank_k, 0), D);
  u.rv = min(max(blk.rank_v, 0), D);
  u.rk16 = (u.r + 15) & ~15;
  u.npairs = (u.r + 63) >> 6;
  u.ntv = (u.rv + 15) >> 4;
  const int r = u.r, rv = u.rv, T = u.T;
  const int64_t head =
      (int64_t)T * u.rk16 + (int64_t)rv * u.ld + 2 * (int64_t)(r + rv) * D + ((8 * (r + rv) + 15) & ~15);
  u.Uk = reinterpret_cast<const uint8_t*>(p.pool) + blk.off + g * head;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(u.Uk + (int64_t)T * u.rk16);
  u.Uv = reinterpret_cast<const uint8_t*>(W + (size_t)r * D);
  const uint16_t* Wp = reinterpret_cast<const uint16_t*>(u.Uv + (size_t)rv * u.ld);
  const float* sbk = reinterpret_cast<const float*>(Wp + (size_t)rv * D);
  const float* sbv = sbk + 2 * r;
  const uint16_t* qh = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)i * p.n_q_heads + g * G) * D;
  float* pf = reinterpret_cast<float*>(lds);          // p' [rank][8 heads]
  float* zs = reinterpret_cast<float*>(lds + 1024);   // z  [rank][8 heads]
  float* abv = reinterpret_cast<float*>(lds + 2048);  // (a', b') of the value rows, after the projection
  const bool small = u.npairs <= 1 && u.ntv <= 4;

  // the value rows' (a', b') go out before the projection
  f32x4_t abv_v = {0.f, 0.f, 0.f, 0.f};   // rows 2 lane, 2 lane + 1
  if (2 * lane < rv) abv_v = *reinterpret_cast<const f32x4_t*>(sbv + 4 * min(lane, (rv - 1) >> 1));

  // ---- p' = p a and C = sum p b (fp32)
  float C[G];
#pragma unroll
  for (int h = 0; h < G; ++h) C[h] = 0.f;
  float mx = 0.f;
  if (r > 0) {
    const f32x2_t ab0 = *reinterpret_cast<const f32x2_t*>(sbk + 2 * min(lane, r - 1));
    f32x2_t ab1 = {0.f, 0.f};
    if (D > 64) ab1 = *reinterpret_cast<const f32x2_t*>(sbk + 2 * min(lane + 64, r - 1));
    mfma_project_q<D, G>(W, qh, r, p.scale_log2, pf, lane);
    wave_lds_fence();
    const bool has0 = lane < r, has1 = D > 64 && lane + 64 < r;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float c = 0.f;
      if (has0) {
        const float x = pf[lane * 8 + h];
        c = x * ab0[1];
        pf[lane * 8 + h] = x * ab0[0];
        mx = fmaxf(mx, fabsf(x * ab0[0]));
      }
      if (has1) {
        const float x = pf[(lane + 64) * 8 + h];
        c = fmaf(x, ab1[1], c);
        pf[(lane + 64) * 8 + h] = x * ab1[0];
        mx = fmaxf(mx, fabsf(x * ab1[0]));
      }
      C[h] = wave_sum(c);
    }
    mx = wave_max(mx);
  }
  // (a', b') of the value rows to LDS (the projection's q staging area is free now)
  if (2 * lane < rv) *reinterpret_cast<f32x4_t*>(abv + 4 * lane) = abv_v;
  wave_lds_fence();
  // sc = 2^(13 - e) with mx < 2^e: the largest |p' sc| stays below 2^13
  const int ex = mx > 0.f ? min(max(ilogbf(mx) + 1, -100), 100) : 0;
  const float sc = ldexpf(1.f, 13 - ex), inv_sc = ldexpf(1.f, ex - 13);
  float Cl = C[0];
#pragma unroll
  for (int h = 1; h < G; ++h) Cl = (u.col == h) ? C[h] : Cl;
  if (u.col >= G) Cl = 0.f;

  float m_run = kNegInf, l_run = 0.f;
  if (small)
    q8_body<1, 4, 2, G>(u, pf, abv, zs, Cl, sc, inv_sc, m_run, l_run);
  else
    q8_body<2, 8, 1, G>(u, pf, abv, zs, Cl, sc, inv_sc, m_run, l_run);
  wave_lds_fence();
  store_zwp<D, G>(p, unit, Wp, rv, zs, m_run, l_run, lane);
}

#include "decode_kivi.inc"

// ---------------------------------------------------------------------------
// fp32 storage (small workloads; same structure, plain FMA)
// ---------------------------------------------------------------------------
template <int D, int G, bool RAGGED>
__device__ __forceinline__ void f32_tiles(const float* Ut, const float* Upt, int ld, int T, int r,
                                          int rv, const float* pf, float (&m_run)[G],
                                          float (&l_run)[G], float* zl, int lane) {
  using S = Shape<D, G>;
  constexpr int R = S::R;
  for (int t0 = 0; t0 < T; t0 += 512) {
    const int tc0 = t0 + lane * 4, tc1 = t0 + 256 + lane * 4;
    const bool ok0 = tc0 < T, ok1 = tc1 < T;
    float s[8][G];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int h = 0; h < G; ++h) s[e][h] = 0.f;
    for (int k = 0; k < r; ++k) {
      const float* row = Ut + (size_t)k * ld;
      f32x4_t u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
      if (ok0) u0 = ld16f(row + tc0);
      if (ok1) u1 = ld16f(row + tc1);
      const f32x4_t pq0 = *reinterpret_cast<const f32x4_t*>(pf + k * 8);
      const f32x4_t pq1 = *reinterpret_cast<const f32x4_t*>(pf + k * 8 + 4);
      const float pp[8] = {pq0[0], pq0[1], pq0[2], pq0[3], pq1[0], pq1[1], pq1[2], pq1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s[e][h] = fmaf(u0[e], pp[h], s[e][h]);
          s[4 + e][h] = fmaf(u1[e], pp[h], s[4 + e][h]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = (e < 4 ? tc0 : tc1) + (e & 3);
      if (tok >= T) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[e][h] = kNegInf;
      }
    }
    float ex[8][G];
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e][h]);
      mx = wave_max(mx);
      const float mn = fmaxf(m_run[h], mx);
      alpha[h] = fast_exp2(m_run[h] - mn);
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ex[e][h] = fast_exp2(s[e][h] - mn);
        sum += ex[e][h];
      }
      l_run[h] = l_run[h] * alpha[h] + wave_sum(sum);
      m_run[h] = mn;
    }
    {
      const int hl = lane % G;
      float al = alpha[0];
#pragma unroll
      for (int h = 1; h < G; ++h) al = (hl == h) ? alpha[h] : al;
      for (int gi = 0; gi * R < rv; ++gi) zl[gi * 64 + lane] *= al;
    }
#pragma unroll 1
    for (int gi = 0; gi * R < rv; ++gi) {
      {
        float acc[64];
#pragma unroll
        for (int x = 0; x < 64; ++x) acc[x] = 0.f;
#pragma unroll
        for (int rho = 0; rho < R; ++rho) {
          const int kp = gi * R + rho;
          if (kp < rv) {
            const float* row = Upt + (size_t)kp * ld;
            f32x4_t u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
            if (ok0) u0 = ld16f(row + tc0);
            if (ok1) u1 = ld16f(row + tc1);
            if (RAGGED) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                u0[e] = (tc0 + e < T) ? u0[e] : 0.f;
                u1[e] = (tc1 + e < T) ? u1[e] : 0.f;
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int h = 0; h < G; ++h) {
                acc[rho * G + h] = fmaf(u0[e], ex[e][h], acc[rho * G + h]);
                acc[rho * G + h] = fmaf(u1[e], ex[4 + e][h], acc[rho * G + h]);
              }
          }
        }
        zl[gi * 64 + lane] += reduce_transpose64(acc, lane);
      }
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void block_unit_f32(const DecodeParams& p, int i, int g, int unit,
                                               const milo_block& blk, uint32_t* lds) {
  using S = Shape<D, G>;
  constexpr int R = S::R, NG = S::NG, JPL = S::JPL;
  const int lane = threadIdx.x;
  const int T = max(blk.n_tok, 0);
  const int ld = blk.ld_tok;
  const int r = min(max(blk.rank_k, 0), D), rv = min(max(blk.rank_v, 0), D);
  const float* Ut = reinterpret_cast<const float*>(p.pool) + blk.off + (int64_t)g * (r + rv) * (ld + D);
  const float* W = Ut + (size_t)r * ld;
  const float* Upt = W + (size_t)r * D;
  const float* Wp = Upt + (size_t)rv * ld;
  const float* qh = reinterpret_cast<const float*>(p.q) + ((int64_t)i * p.n_q_heads + g * G) * D;

  // p[k][h] (fp32) for rows k = lane, lane + 64
  float* pf = reinterpret_cast<float*>(lds);
  {
    float pa[G], pb[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { pa[h] = 0.f; pb[h] = 0.f; }
    const bool has_a = lane < r, has_b = (D > 64) && (lane + 64 < r);
    for (int jc = 0; jc < D / 4; ++jc) {
      f32x4_t wa = {0.f, 0.f, 0.f, 0.f}, wb = {0.f, 0.f, 0.f, 0.f};
      if (has_a) wa = ld16f(W + (size_t)lane * D + jc * 4);
      if (has_b) wb = ld16f(W + (size_t)(lane + 64) * D + jc * 4);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const f32x4_t qv = ld16f(qh + h * D + jc * 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pa[h] = fmaf(wa[w], qv[w], pa[h]);
          pb[h] = fmaf(wb[w], qv[w], pb[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pf[lane * 8 + h] = pa[h] * p.scale_log2;
      if (D > 64) pf[(lane + 64) * 8 + h] = pb[h] * p.scale_log2;
    }
  }
  __syncthreads();

  float* zl = reinterpret_cast<float*>(lds + 1024);
  float m_run[G], l_run[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m_run[h] = kNegInf; l_run[h] = 0.f; }
  for (int gi = 0; gi < NG; ++gi) zl[gi * 64 + lane] = 0.f;
  if (T & 3)
    f32_tiles<D, G, true>(Ut, Upt, ld, T, r, rv, pf, m_run, l_run, zl, lane);
  else
    f32_tiles<D, G, false>(Ut, Upt, ld, T, r, rv, pf, m_run, l_run, zl, lane);

  __syncthreads();
  float o[G][JPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) o[h][jj] = 0.f;
  for (int kp = 0; kp < rv; ++kp) {
    const int gi = kp / R, rho = kp - gi * R;
    const float* zp = zl + gi * 64 + rho * G;
    float wv[JPL];
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) wv[jj] = Wp[(size_t)kp * D + lane * JPL + jj];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float z = zp[h];
#pragma unroll
      for (int jj = 0; jj < JPL; ++jj) o[h][jj] = fmaf(z, wv[jj], o[h][jj]);
    }
  }
  float* po = p.part.o + (size_t)unit * G * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) po[h * D + lane * JPL + jj] = o[h][jj];
#pragma unroll
  for (int h = 0; h < G; ++h)
    if (lane == h) {
      p.part.ml[((size_t)unit * G + h) * 2 + 0] = m_run[h];
      p.part.ml[((size_t)unit * G + h) * 2 + 1] = l_run[h];
    }
}

// ---------------------------------------------------------------------------
// dense tail: K_t, V_t token-major [tail_cap][D]; every token < tail_len is
// visible to the decode query.  Lane t scores token t of a 64-token tile.
// ---------------------------------------------------------------------------
template <int D, int G, int DT>
__device__ __forceinline__ void tail_unit(const DecodeParams& p, int i, int g, int unit,
                                          uint32_t* lds) {
  constexpr int JPL = D / 64;
  const int lane = threadIdx.x;
  const int cap = p.tail_cap;
  const int L = cap > 0 ? min(max(p.tail_len[i], 0), cap) : 0;
  const size_t kv_off = ((size_t)i * p.n_kv_heads + g) * (size_t)cap * D;
  float m_run[G], l_run[G], o[G][JPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) o[h][jj] = 0.f;
  }
  float* el = reinterpret_cast<float*>(lds);   // [64 tokens][8 heads]
  // bf16: q of the group staged in LDS (read back as broadcasts)
  uint16_t* ql = reinterpret_cast<uint16_t*>(lds + 2048);
  if (DT != MILO_F32 && L > 0) {
    constexpr int NQ = G * D / 8;
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)i * p.n_q_heads + g * G) * D;
    if (lane < NQ) *reinterpret_cast<u32x4_t*>(ql + lane * 8) = ld16(qh + lane * 8);
    if (lane + 64 < NQ) *reinterpret_cast<u32x4_t*>(ql + (lane + 64) * 8) = ld16(qh + (lane + 64) * 8);
    wave_lds_fence();
  }
  for (int t0 = 0; t0 < L; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < L;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
    const int tk = min(t, L - 1);   // lanes past the end re-read the last token (masked)
    if (DT != MILO_F32) {
      // the whole key row of the lane's token in flight at once
      const uint16_t* K = reinterpret_cast<const uint16_t*>(p.k_tail) + kv_off + (size_t)tk * D;
      u32x4_t kv[D / 8];
#pragma unroll
      for (int jc = 0; jc < D / 8; ++jc) kv[jc] = ld16(K + jc * 8);
#pragma unroll
      for (int jc = 0; jc < D / 8; ++jc)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(ql + h * D + jc * 8);
#pragma unroll
          for (int w = 0; w < 4; ++w) s[h] = dot2bf(kv[jc][w], qv[w], s[h]);
        }
    } else {
      const float* K = reinterpret_cast<const float*>(p.k_tail) + kv_off + (size_t)tk * D;
      const float* qh = reinterpret_cast<const float*>(p.q) + ((int64_t)i * p.n_q_heads + g * G) * D;
#pragma unroll 4
      for (int jc = 0; jc < D / 4; ++jc) {
        const f32x4_t kv = ld16f(K + jc * 4);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const f32x4_t qv = ld16f(qh + h * D + jc * 4);
#pragma unroll
          for (int w = 0; w < 4; ++w) s[h] = fmaf(kv[w], qv[w], s[h]);
        }
      }
    }
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sv = valid ? s[h] * p.scale_log2 : kNegInf;
      const float mx = wave_max(sv);
      const float mn = fmaxf(m_run[h], mx);
      alpha[h] = fast_exp2(m_run[h] - mn);
      const float ev = fast_exp2(sv - mn);
      l_run[h] = l_run[h] * alpha[h] + wave_sum(ev);
      m_run[h] = mn;
      el[lane * 8 + h] = ev;
#pragma unroll
      for (int jj = 0; jj < JPL; ++jj) o[h][jj] *= alpha[h];
    }
    wave_lds_fence();
    // o~ += e^T V over the tile, eight token rows of V in flight per step
    constexpr int kVRows = 8;
    const int nt = min(64, L - t0);
    for (int tt0 = 0; tt0 < nt; tt0 += kVRows) {
      float vv[kVRows][JPL];
#pragma unroll
      for (int j = 0; j < kVRows; ++j) {
        const size_t row = kv_off + (size_t)(t0 + min(tt0 + j, nt - 1)) * D;
        if (DT != MILO_F32) {
          const uint16_t* V = reinterpret_cast<const uint16_t*>(p.v_tail) + row;
          if (JPL == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(V + 2 * lane);
            vv[j][0] = bf_lo(w);
            vv[j][JPL - 1] = bf_hi(w);
          } else {
            vv[j][0] = __uint_as_float((uint32_t)V[lane] << 16);
          }
        } else {
          const float* V = reinterpret_cast<const float*>(p.v_tail) + row;
#pragma unroll
          for (int jj = 0; jj < JPL; ++jj) vv[j][jj] = V[lane * JPL + jj];
        }
      }
#pragma unroll
      for (int j = 0; j < kVRows; ++j) {
        if (tt0 + j < nt) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float ev = el[(tt0 + j) * 8 + h];
#pragma unroll
            for (int jj = 0; jj < JPL; ++jj) o[h][jj] = fmaf(ev, vv[j][jj], o[h][jj]);
          }
        }
      }
    }
    wave_lds_fence();
  }
  float* po = p.part.o + (size_t)unit * G * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) po[h * D + lane * JPL + jj] = o[h][jj];
#pragma unroll
  for (int h = 0; h < G; ++h)
    if (lane == h) {
      p.part.ml[((size_t)unit * G + h) * 2 + 0] = m_run[h];
      p.part.ml[((size_t)unit * G + h) * 2 + 1] = l_run[h];
    }
}

template <int D, int G, int DT>
__device__ __forceinline__ void decode_wave(const DecodeParams& p, uint32_t* lds) {
  const int S = p.max_blocks + 1;
  const int unit = p.unit_order ? p.unit_order[blockIdx.x] : (int)blockIdx.x;
  if ((unsigned)unit >= (unsigned)(p.batch * p.n_kv_heads * S)) return;   // not a unit index
  const int slot = unit % S;
  const int ig = unit / S;
  const int g = ig % p.n_kv_heads, i = ig / p.n_kv_heads;
  if (slot == p.max_blocks) {
    tail_unit<D, G, DT>(p, i, g, unit, lds);
    return;
  }
  const int b0 = p.seq_blocks[i];
  const int nb = min(max(p.seq_blocks[i + 1] - b0, 0), p.max_blocks);
  if (slot >= nb) return;
  const milo_block blk = p.blocks[b0 + slot];
  if constexpr (DT == MILO_BF16)
    block_unit_bf16<D, G>(p, i, g, unit, blk, lds);
  else if constexpr (DT == MILO_BF16_Q8)
    block_unit_q8<D, G>(p, i, g, unit, blk, lds);
  else if constexpr (DT == MILO_BF16_KV4)
    block_unit_kivi<D, G, 4>(p, i, g, unit, blk, lds);
  else if constexpr (DT == MILO_BF16_KV2)
    block_unit_kivi<D, G, 2>(p, i, g, unit, blk, lds);
  else
    block_unit_f32<D, G>(p, i, g, unit, blk, lds);
}

// bf16 storage: the register budget is set to two waves per SIMD (the
// allocator fits every group size without spills).
template <int D, int G, int DT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void milo_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
  decode_wave<D, G, DT>(p, lds);
}

// fp32 storage
template <int D, int G>
__global__ __launch_bounds__(64) void milo_decode_f32_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
  decode_wave<D, G, MILO_F32>(p, lds);
}

// The 8-bit kernel holds two chunks of code loads in flight; its register
// budget is set to two waves per SIMD (the allocator fits it without spills).
template <int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void milo_decode_q8_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
  decode_wave<D, G, MILO_BF16_Q8>(p, lds);
}

// The KIVI-style kernel holds one or two chunks of loads in flight, with the
// same register budget.
template <int D, int G, int DT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void milo_decode_kv_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
  decode_wave<D, G, DT>(p, lds);
}

// Plain launch, or with the caller's timing events attached to the dispatch.
template <typename K>
void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, LaunchEvents ev, const DecodeParams& p) {
  if (ev.start && ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, p);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, p);
}

template <int D, int G, int DT>
void launch_decode_g(const DecodeParams& p, dim3 grid, hipStream_t s, LaunchEvents ev) {
  if constexpr (DT == MILO_BF16_Q8)
    launch_timed(milo_decode_q8_kernel<D, G>, grid, dim3(64), s, ev, p);
  else if constexpr (DT == MILO_BF16_KV4 || DT == MILO_BF16_KV2)
    launch_timed(milo_decode_kv_kernel<D, G, DT>, grid, dim3(64), s, ev, p);
  else if constexpr (DT == MILO_F32)
    launch_timed(milo_decode_f32_kernel<D, G>, grid, dim3(64), s, ev, p);
  else
    launch_timed(milo_decode_kernel<D, G, DT>, grid, dim3(64), s, ev, p);
}

template <int D, int DT>
hipError_t launch_decode_dg(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev) {
  const int64_t units = decode_units(p.batch, p.n_kv_heads, p.max_blocks);
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)units);
  switch (group) {
#define MILO_G(GG) \
  case GG: launch_decode_g<D, GG, DT>(p, grid, s, ev); break;
    MILO_G(1) MILO_G(2) MILO_G(3) MILO_G(4) MILO_G(5) MILO_G(6) MILO_G(7) MILO_G(8)
#undef MILO_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// One translation unit per (dtype, head_dim): compiled with
// -DMILO_INST_DT=<0|1|2> -DMILO_INST_D=<64|128>.
#define MILO_CAT2(a, b, c) launch_decode_##a##_##b##_##c
#define MILO_CAT(a, b, c) MILO_CAT2(a, b, c)
hipError_t MILO_CAT(dt, MILO_INST_DT, MILO_INST_D)(const DecodeParams& p, int group, hipStream_t s, LaunchEvents ev) {
  return launch_decode_dg<MILO_INST_D, MILO_INST_DT>(p, group, s, ev);
}

}  // namespace milo
