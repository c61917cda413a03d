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
//     row segments); each row of U^T is unpacked to fp32 and met with fp32
//     p held in LDS (broadcast reads), G FMAs per element;
//   - values: the same lane/token ownership; e is packed to bf16 token pairs
//     against rows of U'^T; per-lane partial z of up to 64 (row, head) slots
//     are summed across the wave by one transposing butterfly.
//   - o~ += z W' is applied per row group as soon as the group's z is
//     reduced; the group's W' rows load with its U'^T rows, so no memory
//     round trip is left after the last group.
// The U^T and U'^T streams are read once and wave-coalesced, so they are
// loaded non-temporally.  W is read lane-per-row, all of the unit's rows in
// flight at once (one memory round trip).  A unit is one wave, so LDS
// hand-offs between its lanes need no barrier (a barrier would also wait
// for every load in flight).
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kLdsWords = 2560;   // p (4 KB) | z partials (4 KB) | q of the group (2 KB)
constexpr float kNegInf = -__builtin_huge_valf();

template <int D, int G>
struct Shape {
  static constexpr int R = (64 / G < 12) ? 64 / G : 12;  // value rows per butterfly group
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

// p = scale*log2(e) * W q for the G heads, fp32; lane k owns rows k and k+64
// (the second only when r > 64).  q is staged in LDS (ql) and read back as
// broadcasts; every W load of the lane is issued before the first product,
// so the projection costs one memory round trip.  q and W are bf16, so the
// dot2 products are exact.  Rows are clamped to r-1; rows >= r are never
// read from pf.  Requires r >= 1.
template <int D, int G>
__device__ __forceinline__ void bf16_project_q(const uint16_t* W, const uint16_t* qh, int r,
                                               float scale_log2, float* pf, uint16_t* ql, int lane) {
  constexpr int NC = D / 8, NQ = G * NC;   // 16-byte chunks per row; q chunks of the group
  u32x4_t q0 = {0u, 0u, 0u, 0u}, q1 = {0u, 0u, 0u, 0u};
  if (lane < NQ) q0 = ld16(qh + lane * 8);
  if (lane + 64 < NQ) q1 = ld16(qh + (lane + 64) * 8);
  const bool two = D > 64 && r > 64;
  u32x4_t wa[NC], wb[NC];
  const uint16_t* wa_row = W + (size_t)min(lane, r - 1) * D;
  const uint16_t* wb_row = W + (size_t)min(lane + 64, r - 1) * D;
#pragma unroll
  for (int jc = 0; jc < NC; ++jc) wa[jc] = ld16(wa_row + jc * 8);
  if (two) {
#pragma unroll
    for (int jc = 0; jc < NC; ++jc) wb[jc] = ld16(wb_row + jc * 8);
  }
  if (lane < NQ) *reinterpret_cast<u32x4_t*>(ql + lane * 8) = q0;
  if (lane + 64 < NQ) *reinterpret_cast<u32x4_t*>(ql + (lane + 64) * 8) = q1;
  wave_lds_fence();
  float pa[G], pb[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { pa[h] = 0.f; pb[h] = 0.f; }
#pragma unroll
  for (int jc = 0; jc < NC; ++jc)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(ql + h * D + jc * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) pa[h] = dot2bf(wa[jc][w], qv[w], pa[h]);
    }
#pragma unroll
  for (int h = 0; h < G; ++h) pf[lane * 8 + h] = pa[h] * scale_log2;
  if (two) {
#pragma unroll
    for (int jc = 0; jc < NC; ++jc)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(ql + h * D + jc * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) pb[h] = dot2bf(wb[jc][w], qv[w], pb[h]);
      }
#pragma unroll
    for (int h = 0; h < G; ++h) pf[(lane + 64) * 8 + h] = pb[h] * scale_log2;
  }
}

constexpr int kRowsPerStep = 4;   // U^T rows per prefetch step of the score loop

// Loads rows k0 .. k0+3 of U^T (clamped to r-1) at the lane's two chunks.
__device__ __forceinline__ void load_rows4(const uint16_t* Ut, int ld, int k0, int r, int tq0,
                                           int tq1, u32x4_t (&A)[kRowsPerStep],
                                           u32x4_t (&B)[kRowsPerStep]) {
#pragma unroll
  for (int j = 0; j < kRowsPerStep; ++j) {
    const uint16_t* row = Ut + (size_t)min(k0 + j, r - 1) * ld;
    A[j] = ld16_stream(row + tq0);
    B[j] = ld16_stream(row + tq1);
  }
}

template <int G>
__device__ __forceinline__ void score_rows4(const u32x4_t (&A)[kRowsPerStep],
                                            const u32x4_t (&B)[kRowsPerStep], int k0, int r,
                                            const float* pf, float (&s)[16][G]) {
#pragma unroll
  for (int j = 0; j < kRowsPerStep; ++j) {
    if (k0 + j < r) {
      const f32x4_t pq0 = *reinterpret_cast<const f32x4_t*>(pf + (k0 + j) * 8);
      const f32x4_t pq1 = *reinterpret_cast<const f32x4_t*>(pf + (k0 + j) * 8 + 4);
      const float pp[8] = {pq0[0], pq0[1], pq0[2], pq0[3], pq1[0], pq1[1], pq1[2], pq1[3]};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a0 = bf_lo(A[j][w]), a1 = bf_hi(A[j][w]);
        const float b0 = bf_lo(B[j][w]), b1 = bf_hi(B[j][w]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s[2 * w][h] = fmaf(a0, pp[h], s[2 * w][h]);
          s[2 * w + 1][h] = fmaf(a1, pp[h], s[2 * w + 1][h]);
          s[8 + 2 * w][h] = fmaf(b0, pp[h], s[8 + 2 * w][h]);
          s[8 + 2 * w + 1][h] = fmaf(b1, pp[h], s[8 + 2 * w + 1][h]);
        }
      }
    }
  }
}

// One 1024-token tile at a time: scores, online softmax, then per group of
// R rows of U'^T the group's z = e^T U' and at once o~ += z W' for those
// rows (W' rows load with the group), so no pass over W' is left at the end.
// o~ is rescaled with the softmax like l.
template <int D, int G, bool RAGGED>
__device__ __forceinline__ void bf16_tiles(const uint16_t* Ut, const uint16_t* Upt,
                                           const uint16_t* Wp, int ld, int T, int r, int rv,
                                           const float* pf, float (&m_run)[G], float (&l_run)[G],
                                           float (&o)[G][D / 64], float* zs, int lane) {
  using S = Shape<D, G>;
  constexpr int R = S::R, JPL = S::JPL;
  for (int t0 = 0; t0 < T; t0 += 1024) {
    const int tc0 = t0 + lane * 8, tc1 = t0 + 512 + lane * 8;
    const bool ok0 = tc0 < T, ok1 = tc1 < T;
    // A lane whose chunk lies past the block end reads the tile's first
    // chunk instead (always in bounds) and its tokens are masked below.
    const int tq0 = ok0 ? tc0 : t0, tq1 = ok1 ? tc1 : t0;

    // ---- scores s[c*8+e][h] for token tc_c + e: U rows unpacked to fp32
    // and met with fp32 p (bf16 rounding of p would cost ~1% on sharp softmax)
    float s[16][G];
#pragma unroll
    for (int e = 0; e < 16; ++e)
#pragma unroll
      for (int h = 0; h < G; ++h) s[e][h] = 0.f;
    if (r > 0) {
      u32x4_t A0[kRowsPerStep], B0[kRowsPerStep], A1[kRowsPerStep], B1[kRowsPerStep];
      load_rows4(Ut, ld, 0, r, tq0, tq1, A0, B0);
      for (int k0 = 0; k0 < r; k0 += 2 * kRowsPerStep) {
        if (k0 + kRowsPerStep < r) load_rows4(Ut, ld, k0 + kRowsPerStep, r, tq0, tq1, A1, B1);
        score_rows4<G>(A0, B0, k0, r, pf, s);
        if (k0 + 2 * kRowsPerStep < r) load_rows4(Ut, ld, k0 + 2 * kRowsPerStep, r, tq0, tq1, A0, B0);
        if (k0 + kRowsPerStep < r) score_rows4<G>(A1, B1, k0 + kRowsPerStep, r, pf, s);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tok = (e < 8 ? tc0 : tc1) + (e & 7);
      if (tok >= T) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[e][h] = kNegInf;
      }
    }

    // ---- online softmax statistics; e packed to bf16 token pairs
    uint32_t e2[2][4][G];
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e][h]);
      mx = wave_max(mx);
      const float mn = fmaxf(m_run[h], mx);
      alpha[h] = fast_exp2(m_run[h] - mn);
      float sum = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float x0 = fast_exp2(s[c * 8 + 2 * w][h] - mn);
          const float x1 = fast_exp2(s[c * 8 + 2 * w + 1][h] - mn);
          sum += x0 + x1;
          e2[c][w][h] = pack_bf16(x0, x1);
        }
      l_run[h] = l_run[h] * alpha[h] + wave_sum(sum);
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
    u32x4_t mask0 = {~0u, ~0u, ~0u, ~0u}, mask1 = {~0u, ~0u, ~0u, ~0u};
    if (RAGGED) {
      const int n0 = ok0 ? T - tc0 : 0, n1 = ok1 ? T - tc1 : 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mask0[w] = (2 * w < n0 ? 0xffffu : 0u) | (2 * w + 1 < n0 ? 0xffff0000u : 0u);
        mask1[w] = (2 * w < n1 ? 0xffffu : 0u) | (2 * w + 1 < n1 ? 0xffff0000u : 0u);
      }
    }
#pragma unroll 1
    for (int gi = 0; gi * R < rv; ++gi) {
      u32x4_t U0[R], U1[R];
      uint32_t wr[R];   // the lane's JPL columns of the group's W' rows
#pragma unroll
      for (int rho = 0; rho < R; ++rho) {
        const int k = min(gi * R + rho, rv - 1);
        const uint16_t* row = Upt + (size_t)k * ld;
        U0[rho] = ld16_stream(row + tq0);
        U1[rho] = ld16_stream(row + tq1);
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
        u32x4_t u0 = U0[rho], u1 = U1[rho];
        if (RAGGED) { u0 &= mask0; u1 &= mask1; }
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[rho * G + h] = dot2bf(u0[w], e2[0][w][h], acc[rho * G + h]);
            acc[rho * G + h] = dot2bf(u1[w], e2[1][w][h], acc[rho * G + h]);
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
    }
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
  if (r > 0) bf16_project_q<D, G>(W, qh, r, p.scale_log2, pf, reinterpret_cast<uint16_t*>(lds + 2048), lane);
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

  if (T & 7)
    bf16_tiles<D, G, true>(Ut, Upt, Wp, ld, T, r, rv, pf, m_run, l_run, o, zs, lane);
  else
    bf16_tiles<D, G, false>(Ut, Upt, Wp, ld, T, r, rv, pf, m_run, l_run, o, zs, lane);

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
// 8-bit token factors (MILO_BF16_Q8): row k of U^T / U'^T holds codes c with
// x = a_k c + b_k.  Folded into the absorbed order:
//   s_t = sum_k p_k x_kt  = sum_k (p_k a_k) c_kt + C,   C = sum_k p_k b_k
//   z_k = sum_t e_t x'_kt = a'_k sum_t e_t c'_kt + b'_k E,   E = sum_t e_t
// The scores keep the fp32 path of bf16 storage (a code converts to fp32 in
// one instruction).  For the values e is rounded to fp16 pairs, and a byte
// permute with the constant 0x64 turns four codes into two fp16 pairs of
// 1024 + c (exact: fp16 spacing is 1 on [1024, 2048)), so one dot2 per
// token pair and head accumulates sum_t e_t (1024 + c); the 1024 E it adds
// is taken off with E summed from the same fp16 e, which also feeds l.
// A lane owns 16 consecutive tokens (one 16-byte load per row) of a
// 1024-token tile.  Codes can not be NaN, so padding needs no mask: tokens
// past the block end have e = 0.
// ---------------------------------------------------------------------------

constexpr int kQ8RowsPerStep = 8;   // U^T rows per prefetch step of the score loop
constexpr uint32_t kF16Ones = 0x3C003C00u;   // fp16 pair (1, 1)
constexpr uint32_t kF16Magic = 0x64646464u;  // high byte of fp16 1024 + c, c < 256

// fp16 pairs (1024 + c0, 1024 + c1) and (1024 + c2, 1024 + c3) of four codes
__device__ __forceinline__ uint32_t q8_pair_lo(uint32_t c) { return __builtin_amdgcn_perm(kF16Magic, c, 0x04010400u); }
__device__ __forceinline__ uint32_t q8_pair_hi(uint32_t c) { return __builtin_amdgcn_perm(kF16Magic, c, 0x04030402u); }

__device__ __forceinline__ void q8_load_rows(const uint8_t* Uc, int ld, int k0, int r, int tq,
                                             u32x4_t (&A)[kQ8RowsPerStep]) {
#pragma unroll
  for (int j = 0; j < kQ8RowsPerStep; ++j) A[j] = ld16_stream(Uc + (size_t)min(k0 + j, r - 1) * ld + tq);
}

template <int G>
__device__ __forceinline__ void q8_score_rows(const u32x4_t (&A)[kQ8RowsPerStep], int k0, int r,
                                              const float* pf, float (&s)[16][G]) {
#pragma unroll
  for (int j = 0; j < kQ8RowsPerStep; ++j) {
    if (k0 + j < r) {
      const f32x4_t pq0 = *reinterpret_cast<const f32x4_t*>(pf + (k0 + j) * 8);
      const f32x4_t pq1 = *reinterpret_cast<const f32x4_t*>(pf + (k0 + j) * 8 + 4);
      const float pp[8] = {pq0[0], pq0[1], pq0[2], pq0[3], pq1[0], pq1[1], pq1[2], pq1[3]};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = A[j][w];
        const float c[4] = {(float)(x & 0xffu), (float)((x >> 8) & 0xffu), (float)((x >> 16) & 0xffu),
                            (float)(x >> 24)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int h = 0; h < G; ++h) s[4 * w + e][h] = fmaf(c[e], pp[h], s[4 * w + e][h]);
      }
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void q8_tiles(const uint8_t* Uc, const uint8_t* Upc, const uint16_t* Wp,
                                         const float* sbv, int ld, int T, int r, int rv, const float* pf,
                                         const float (&C)[G], float (&m_run)[G], float (&l_run)[G],
                                         float (&o)[G][D / 64], float* zs, int lane) {
  using S = Shape<D, G>;
  constexpr int R = S::R, JPL = S::JPL;
  const int hl = lane % G;   // head of the lane's z slot
  for (int t0 = 0; t0 < T; t0 += 1024) {
    const int tc = t0 + lane * 16;
    // a lane whose chunk lies past the block end reads the tile's first
    // chunk instead (always in bounds); its tokens are masked below
    const int tq = tc < T ? tc : t0;

    float s[16][G];
#pragma unroll
    for (int e = 0; e < 16; ++e)
#pragma unroll
      for (int h = 0; h < G; ++h) s[e][h] = C[h];
    if (r > 0) {
      u32x4_t A0[kQ8RowsPerStep], A1[kQ8RowsPerStep];
      q8_load_rows(Uc, ld, 0, r, tq, A0);
      for (int k0 = 0; k0 < r; k0 += 2 * kQ8RowsPerStep) {
        if (k0 + kQ8RowsPerStep < r) q8_load_rows(Uc, ld, k0 + kQ8RowsPerStep, r, tq, A1);
        q8_score_rows<G>(A0, k0, r, pf, s);
        if (k0 + 2 * kQ8RowsPerStep < r) q8_load_rows(Uc, ld, k0 + 2 * kQ8RowsPerStep, r, tq, A0);
        if (k0 + kQ8RowsPerStep < r) q8_score_rows<G>(A1, k0 + kQ8RowsPerStep, r, pf, s);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (tc + e >= T) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[e][h] = kNegInf;
      }
    }

    // online softmax; e as fp16 pairs, E (the sum of those fp16 values) per head
    uint32_t e2[8][G];
    float alpha[G], E[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e][h]);
      mx = wave_max(mx);
      const float mn = fmaxf(m_run[h], mx);
      alpha[h] = fast_exp2(m_run[h] - mn);
      float sum = 0.f;
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) {
        e2[pr][h] = pack_f16(fast_exp2(s[2 * pr][h] - mn), fast_exp2(s[2 * pr + 1][h] - mn));
        sum = dot2h(e2[pr][h], kF16Ones, sum);
      }
      E[h] = wave_sum(sum);
      l_run[h] = l_run[h] * alpha[h] + E[h];
      m_run[h] = mn;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int jj = 0; jj < JPL; ++jj) o[h][jj] *= alpha[h];
    float El = E[0];
#pragma unroll
    for (int h = 1; h < G; ++h) El = (hl == h) ? E[h] : El;

    // ---- z per group of R rows of U'^T, then o~ += z W' for the group
#pragma unroll 1
    for (int gi = 0; gi * R < rv; ++gi) {
      u32x4_t U[R];
      uint32_t wr[R];
#pragma unroll
      for (int rho = 0; rho < R; ++rho)
        U[rho] = ld16_stream(Upc + (size_t)min(gi * R + rho, rv - 1) * ld + tq);
#pragma unroll
      for (int rho = 0; rho < R; ++rho) {
        const uint16_t* wrow = Wp + (size_t)min(gi * R + rho, rv - 1) * D;
        wr[rho] = (JPL == 2) ? *reinterpret_cast<const uint32_t*>(wrow + 2 * lane)
                             : (uint32_t)wrow[lane] << 16;
      }
      // (a', b') of the row of the lane's z slot (lanes >= R*G: unused)
      const f32x2_t ab = *reinterpret_cast<const f32x2_t*>(sbv + 2 * min(gi * R + min(lane / G, R - 1), rv - 1));
      float acc[64];
#pragma unroll
      for (int x = 0; x < 64; ++x) acc[x] = 0.f;
#pragma unroll
      for (int rho = 0; rho < R; ++rho) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = q8_pair_lo(U[rho][w]), hi = q8_pair_hi(U[rho][w]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[rho * G + h] = dot2h(lo, e2[2 * w][h], acc[rho * G + h]);
            acc[rho * G + h] = dot2h(hi, e2[2 * w + 1][h], acc[rho * G + h]);
          }
        }
      }
      // lane l ends with sum_t e_t (1024 + c) of slot l = (row rho, head h)
      const float zg = reduce_transpose64(acc, lane);
      if (lane < R * G) zs[(lane / G) * 8 + hl] = fmaf(ab[0], zg - 1024.f * El, ab[1] * El);
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
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void block_unit_q8(const DecodeParams& p, int i, int g, int unit,
                                              const milo_block& blk, uint32_t* lds) {
  constexpr int JPL = D / 64;
  const int lane = threadIdx.x;
  const int T = max(blk.n_tok, 0);
  const int ld = blk.ld_tok;
  const int r = min(max(blk.rank_k, 0), D), rv = min(max(blk.rank_v, 0), D);
  const int64_t head = (int64_t)(r + rv) * (ld + 2 * D) + ((8 * (r + rv) + 15) & ~15);
  const uint8_t* Uc = reinterpret_cast<const uint8_t*>(p.pool) + blk.off + g * head;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(Uc + (size_t)r * ld);
  const uint8_t* Upc = Uc + (size_t)r * ld + (size_t)r * 2 * D;
  const uint16_t* Wp = reinterpret_cast<const uint16_t*>(Upc + (size_t)rv * ld);
  const float* sbk = reinterpret_cast<const float*>(Uc + (int64_t)(r + rv) * (ld + 2 * D));
  const float* sbv = sbk + 2 * r;
  const uint16_t* qh = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)i * p.n_q_heads + g * G) * D;

  float* pf = reinterpret_cast<float*>(lds);
  float C[G];
#pragma unroll
  for (int h = 0; h < G; ++h) C[h] = 0.f;
  if (r > 0) {
    // (a_k, b_k) of the lane's rows, in flight with the projection's loads
    const f32x2_t ab0 = *reinterpret_cast<const f32x2_t*>(sbk + 2 * min(lane, r - 1));
    f32x2_t ab1 = {0.f, 0.f};
    if (D > 64) ab1 = *reinterpret_cast<const f32x2_t*>(sbk + 2 * min(lane + 64, r - 1));
    bf16_project_q<D, G>(W, qh, r, p.scale_log2, pf, reinterpret_cast<uint16_t*>(lds + 2048), lane);
    wave_lds_fence();
    // p_k a_k replaces p_k; C = sum_k p_k b_k
    const bool has0 = lane < r, has1 = D > 64 && lane + 64 < r;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float c = 0.f;
      if (has0) {
        const float x = pf[lane * 8 + h];
        c = x * ab0[1];
        pf[lane * 8 + h] = x * ab0[0];
      }
      if (has1) {
        const float x = pf[(lane + 64) * 8 + h];
        c = fmaf(x, ab1[1], c);
        pf[(lane + 64) * 8 + h] = x * ab1[0];
      }
      C[h] = wave_sum(c);
    }
  }
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

  q8_tiles<D, G>(Uc, Upc, Wp, sbv, ld, T, r, rv, pf, C, m_run, l_run, o, zs, lane);

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
__global__ __launch_bounds__(64) void milo_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
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
  if (DT == MILO_BF16)
    block_unit_bf16<D, G>(p, i, g, unit, blk, lds);
  else if (DT == MILO_BF16_Q8)
    block_unit_q8<D, G>(p, i, g, unit, blk, lds);
  else
    block_unit_f32<D, G>(p, i, g, unit, blk, lds);
}

template <int D, int DT>
hipError_t launch_decode_dg(const DecodeParams& p, int group, hipStream_t s) {
  const int64_t units = decode_units(p.batch, p.n_kv_heads, p.max_blocks);
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)units), block(64);
  switch (group) {
#define MILO_G(GG) \
  case GG: hipLaunchKernelGGL((milo_decode_kernel<D, GG, DT>), grid, block, 0, s, p); break;
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
hipError_t MILO_CAT(dt, MILO_INST_DT, MILO_INST_D)(const DecodeParams& p, int group, hipStream_t s) {
  return launch_decode_dg<MILO_INST_D, MILO_INST_DT>(p, group, s);
}

}  // namespace milo
