// encode.hip -- gfx950 encode step: per-block low-rank factors of the dense
// keys and values of a context.
//
// MILO (summary at paperlayer.ai/abs/2609.29913v1) stores each block's keys
// and values separately as low-rank factors ("4.2 Block-wise Low-Rank
// Compression") at block-specific ranks ("4.3 Dynamic Rank Allocation",
// "4.4 MILO Workflow").  The factorisation is read as the truncated SVD:
// for a block X (T x d), W = the top-r right singular vectors as rows and
// U = X W^T, so that U W is the best rank-r approximation of X.
//
// Two kernels, one workgroup per (block, KV head, K/V) matrix:
//  spectrum  G = X^T X (fp32 sums of exact products), then its symmetric
//            eigen-decomposition in fp32 by Householder reduction to
//            tridiagonal form and implicit QL iterations whose rotations
//            are accumulated into the Householder factor (the scheme of
//            the textbook tred2/tql2 pair, organised for one workgroup;
//            the steps are listed before the kernel).  Output: sigma_i =
//            sqrt(max(lambda_i, 0)) descending and the eigenvectors as
//            rows, sorted the same way (workspace).
//  factors   W = the first r eigenvector rows, U^T = W X^T, written into
//            the pool in the storage type (RNE for bf16), U^T rows
//            zero-padded to ld_tok: bf16 on the matrix cores (W split into
//            bf16 hi + lo), fp32 on the vector ALUs (fp32 sums).
#include "device_common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace milo {

namespace {

constexpr int kEncThreads = 512;
constexpr int kFacTokens = 64;     // tokens per staged chunk in the factors kernel

// 8 consecutive elements of a dense array as fp32 (16-byte aligned).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&x)[8]) {
  if (DT == MILO_BF16) {
    const u32x4_t w = ld16(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf_lo(w[i]);
      x[2 * i + 1] = bf_hi(w[i]);
    }
  } else {
    const float* f = reinterpret_cast<const float*>(base) + elem;
    const f32x4_t a = ld16f(f), b = ld16f(f + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}

// Four consecutive elements (aligned to 4 elements) in the storage type.
template <int DT>
__device__ __forceinline__ void store4(void* base, int64_t elem, const float (&x)[4]) {
  if (DT == MILO_BF16) {
    uint32_t* p = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(base) + elem);
    p[0] = pack_bf16(x[0], x[1]);
    p[1] = pack_bf16(x[2], x[3]);
  } else {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + elem) = f32x4_t{x[0], x[1], x[2], x[3]};
  }
}

template <int DT>
__device__ __forceinline__ void store1(void* base, int64_t elem, float x) {
  if (DT == MILO_BF16) {
    const uint32_t w = pack_bf16(x, 0.f);
    reinterpret_cast<uint16_t*>(base)[elem] = (uint16_t)(w & 0xffffu);
  } else {
    reinterpret_cast<float*>(base)[elem] = x;
  }
}

// Matrix m = (b * n_kv_heads + g) * 2 + kv: its block, head, K/V and the
// token range clamped to the dense arrays.
struct EncMat {
  int b, g, kv, T;
  int64_t row0;   // element index of the block's first token row in k or v
};
__device__ __forceinline__ EncMat enc_mat(const EncodeParams& p, int m, int D) {
  EncMat e;
  e.kv = m & 1;
  const int bg = m >> 1;
  e.g = bg % p.n_kv_heads;
  e.b = bg / p.n_kv_heads;
  const int64_t start = p.tok_start[e.b];
  const int n = max(p.blocks[e.b].n_tok, 0);
  e.T = (start >= 0 && start <= p.n_tokens) ? (int)min<int64_t>(n, p.n_tokens - start) : 0;
  e.row0 = ((int64_t)e.g * p.n_tokens + (e.T > 0 ? start : 0)) * D;
  return e;
}

// ---------------------------------------------------------------------------
// Spectrum.  One 256-thread workgroup per matrix, about 72 KB of LDS, so two
// matrices share a CU.  Phases:
//  1. G = X^T X: bf16 inputs on v_mfma_f32_16x16x32_bf16 (exact products,
//     fp32 sums) from token chunks staged transposed in LDS; fp32 inputs on
//     the vector ALUs.  G is mirrored from its upper triangle (exactly
//     symmetric) and scaled by a power of two (exact) to trace ~ 1.
//  2. Householder reduction to tridiagonal form (d, e), in place: step k
//     annihilates row k right of the superdiagonal with H = I - tau v v^T
//     (v_0 = 1), whose v is kept in that row; the trailing block is updated
//     as A -= v w^T + w v^T, w = p - (tau/2)(p.v) v, p = tau A v.  The row
//     is scaled by a power of two before its norm is taken.
//  3. Q^T = H_{d-3} ... H_1 H_0 accumulated in place (from the last
//     reflector back: Q^T <- Q^T H_k on the trailing block).
//  4. Implicit QL with a Wilkinson-type shift on (d, e) taken in reverse
//     order (the tridiagonal forms of these Gram matrices are graded, large
//     at the top, and QL from the other end needs about a third fewer
//     rotations in the worst case), every plane rotation applied to the rows
//     of Q^T (the columns of Q): one wave per 64 entries of a row runs the
//     same scalar recurrence (each on its own copy of d and e) and rotates
//     its entries of the two rows.
//     e_m counts as zero when |e_m| <= 2^-24 (|d_m| + |d_m+1|) or <= 1e-8
//     trace; at most 30 iterations per eigenvalue.
//  5. sigma_i = sqrt(max(lambda_i, 0)) descending and the eigenvectors (the
//     rows of Q^T) in the same order.
// Rows of the matrix phases are read and written as aligned 16-byte chunks
// (row stride D + 4 floats: eight rows' chunks fall in distinct banks).
// ---------------------------------------------------------------------------
constexpr int kEigThreads = 256;
constexpr int kEigMaxIt = 30;
constexpr float kEigTolRel = 0x1p-24f;
constexpr float kEigTolAbs = 1e-8f;
constexpr int kGramTok = 128;           // tokens per staged chunk (bf16 Gram)
constexpr int kGramXs = kGramTok + 8;   // bf16 per staged row (272 B: 8 rows hit 8 distinct 16-B bank groups)

template <int D>
struct EigSmem {
  static constexpr int S = D + 4;   // row stride of a, in floats
  float a[D * S];                   // X staging, then G, the reflectors and Q^T, then the eigenvectors
  float vb[1][D];                   // v of the current reflector by column (0 left of its block)
  float wb[4][D];                   // w by column, one copy per wave
  float part[2][D];                 // partial row products of the two column halves
  float tau[D];
  f32x2_t de[2][D];                 // (d, e) of the tridiagonal form in reverse order, (d_{D-1-i}, e_{D-2-i});
                                    // one copy per QL wave
  float lam[D];                     // eigenvalues
  int rank[D];
  float trace;
};

// Products that must not be contracted into fused multiply-adds, so that
// A -= v w^T + w v^T stays exactly symmetric.
__device__ __forceinline__ float sym2(float vi, float wj, float wi, float vj) {
  return __fadd_rn(__fmul_rn(vi, wj), __fmul_rn(wi, vj));
}

__device__ __forceinline__ f32x4_t lds4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }
__device__ __forceinline__ void sts4(float* p, const f32x4_t& v) { *reinterpret_cast<f32x4_t*>(p) = v; }

// The trailing block of step k covers columns k+1 .. D-1, walked in
// aligned 4-column chunks from (k+1) & ~3; the first ceil(n/2) of its n
// chunks form half 0, the rest half 1 (at most D/8 each).
struct Halves {
  int c0, n;   // first chunk column, chunk count
};
template <int D>
__device__ __forceinline__ Halves half_of(int k, int hh) {
  const int c0 = (k + 1) & ~3, nt = (D - c0) / 4, n0 = (nt + 1) / 2;
  Halves h;
  h.c0 = hh ? c0 + 4 * n0 : c0;
  h.n = hh ? nt - n0 : n0;
  return h;
}

// G = X^T X for bf16 X on the matrix cores.  Chunks of kGramTok tokens are
// staged as xt[dim][token] (token pairs packed per dword).  Wave w owns the
// 16-row tile rows I = (D/64) w .. +D/64 - 1 and every tile column J; lane l
// of tile (I, J) ends with G[16I + 4(l/16) + v][16J + l%16].
template <int D>
__device__ __forceinline__ void gram_bf16(const uint16_t* x, int64_t row0, int T, EigSmem<D>& sm, int tid) {
  constexpr int NT = D / 16, IPW = NT / 4;
  constexpr int ITEMS = (kGramTok / 2) * (D / 8) / kEigThreads;   // (token pair, 8 dims) items per thread
  static_assert(ITEMS * kEigThreads == (kGramTok / 2) * (D / 8), "staging split");
  uint32_t* xt = reinterpret_cast<uint32_t*>(sm.a);   // [D][kGramXs / 2] dwords
  const int lane = tid & 63, wave = tid >> 6;
  f32x4_t acc[IPW][NT];
#pragma unroll
  for (int i = 0; i < IPW; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t r0[ITEMS], r1[ITEMS];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int it = tid + kEigThreads * u;
      const int tp = it % (kGramTok / 2), cg = it / (kGramTok / 2);
      const int ta = t0 + 2 * tp, tb = ta + 1;
      r0[u] = ta < T ? ld16(x + row0 + (int64_t)ta * D + 8 * cg) : u32x4_t{0u, 0u, 0u, 0u};
      r1[u] = tb < T ? ld16(x + row0 + (int64_t)tb * D + 8 * cg) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  if (T > 0) fetch(0);
  for (int t0 = 0; t0 < T; t0 += kGramTok) {
    __syncthreads();   // the previous chunk's operand reads are done
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int it = tid + kEigThreads * u;
      const int tp = it % (kGramTok / 2), cg = it / (kGramTok / 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xt[(8 * cg + 2 * i) * (kGramXs / 2) + tp] = perm_lo(r0[u][i], r1[u][i]);
        xt[(8 * cg + 2 * i + 1) * (kGramXs / 2) + tp] = perm_hi(r0[u][i], r1[u][i]);
      }
    }
    __syncthreads();
    if (t0 + kGramTok < T) fetch(t0 + kGramTok);
    const int nk = min(kGramTok, T - t0 + 31) / 32;   // K steps holding tokens (the rest of the chunk is zero)
    for (int s = 0; s < nk; ++s) {
      const int off = 16 * s + 4 * (lane >> 4);       // dword offset of the lane's 8 tokens
      u32x4_t bo[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bo[j] = *reinterpret_cast<const u32x4_t*>(xt + (16 * j + (lane & 15)) * (kGramXs / 2) + off);
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int I = IPW * wave + i;
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma32(bo[I], bo[j], acc[i][j]);
      }
    }
  }
  __syncthreads();   // staging reads are done before G overwrites it
  constexpr int S = EigSmem<D>::S;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int I = IPW * wave + i;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) sm.a[(16 * I + 4 * (lane >> 4) + v) * S + 16 * j + (lane & 15)] = acc[i][j][v];
  }
}

// G = X^T X for fp32 X on the vector ALUs: chunks of D tokens staged as
// rows; thread (ti, tj) of a 16 x 16 grid owns a (D/16) x (D/16) tile.
template <int D>
__device__ __forceinline__ void gram_f32(const float* x, int64_t row0, int T, EigSmem<D>& sm, int tid) {
  constexpr int TI = D / 16;
  const int i0 = (tid >> 4) * TI, j0 = (tid & 15) * TI;
  float acc[TI][TI];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j) acc[i][j] = 0.f;
  float* xs = sm.a;   // D token rows x D
  for (int t0 = 0; t0 < T; t0 += D) {
    const int n = min(D, T - t0);
    __syncthreads();
    for (int q = tid; q < D * (D / 4); q += kEigThreads) {
      const int t = q / (D / 4), c = (q % (D / 4)) * 4;
      const f32x4_t v = t < n ? ld16f(x + row0 + (int64_t)(t0 + t) * D + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      sts4(xs + t * D + c, v);
    }
    __syncthreads();
    for (int t = 0; t < n; ++t) {
      float u[TI], w[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) u[i] = xs[t * D + i0 + i];
#pragma unroll
      for (int j = 0; j < TI; ++j) w[j] = xs[t * D + j0 + j];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j) acc[i][j] = fmaf(u[i], w[j], acc[i][j]);
    }
  }
  __syncthreads();
  constexpr int S = EigSmem<D>::S;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j) sm.a[(i0 + i) * S + j0 + j] = acc[i][j];
}

// Householder reduction of the symmetric matrix in sm.a to tridiagonal
// form.  Thread (hh, ii) = (tid / 128, tid % 128) owns row k+1+ii of the
// trailing block over column half hh, as up to 16 aligned chunks held in
// registers between the product and the update of a step.
template <int D>
__device__ __forceinline__ void tridiagonalize(EigSmem<D>& sm, int tid) {
  constexpr int S = EigSmem<D>::S, NC = D / 8;   // chunks per half, at most
  float* A = sm.a;
  const int lane = tid & 63, wave = tid >> 6, hh = tid >> 7, ii = tid & 127;
  auto pvec = [&](int c, float tk) { return tk * (sm.part[0][c] + sm.part[1][c]); };
  for (int k = 0; k < D - 2; ++k) {
    const int m = D - 1 - k;   // trailing size
    if (wave == 0) {
      // reflector from row k, columns k+1 .. D-1 (x_i = A[k][k+1+i])
      const int i0 = lane, i1 = lane + 64;
      float x0 = i0 < m ? A[k * S + k + 1 + i0] : 0.f;
      float x1 = i1 < m ? A[k * S + k + 1 + i1] : 0.f;
      const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      float tk = 0.f, ek = A[k * S + k + 1], v0 = i0 == 0 ? 1.f : 0.f, v1 = 0.f;
      if (amax > 0.f) {
        int ex;
        frexpf(amax, &ex);
        x0 = ldexpf(x0, -ex);   // exact
        x1 = ldexpf(x1, -ex);
        const float alpha = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x0)));
        const float xn2 = wave_sum((i0 == 0 ? 0.f : x0 * x0) + x1 * x1);
        if (xn2 > 0.f) {
          const float beta = -copysignf(sqrtf(alpha * alpha + xn2), alpha);
          tk = (beta - alpha) * __builtin_amdgcn_rcpf(beta);
          const float inv = __builtin_amdgcn_rcpf(alpha - beta);
          v0 = i0 == 0 ? 1.f : x0 * inv;
          v1 = x1 * inv;
          ek = ldexpf(beta, ex);
        }
      }
      // vb by column: v at k+1.., zero left of the block (disjoint stores);
      // v past v_0 is kept in row k
      float* vb = sm.vb[0];
      if (lane < k + 1) vb[lane] = 0.f;
      if (lane + 64 < k + 1) vb[lane + 64] = 0.f;
      if (i0 < m) vb[k + 1 + i0] = v0;
      if (i1 < m) vb[k + 1 + i1] = v1;
      if (i0 > 0 && i0 < m) A[k * S + k + 1 + i0] = v0;
      if (i1 < m) A[k * S + k + 1 + i1] = v1;
      if (lane == 0) {
        sm.tau[k] = tk;
        sm.de[0][D - 1 - k][0] = sm.de[1][D - 1 - k][0] = A[k * S + k];
        sm.de[0][D - 2 - k][1] = sm.de[1][D - 2 - k][1] = ek;
      }
    }
    __syncthreads();
    const float tk = sm.tau[k];
    if (tk == 0.f) continue;   // H = I (uniform)
    const Halves h = half_of<D>(k, hh);
    const bool act = ii < m;
    float* ar = A + (k + 1 + ii) * S + h.c0;
    f32x4_t row[NC];
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      if (q < h.n && act) {
        row[q] = lds4(ar + 4 * q);
        const f32x4_t vq = lds4(sm.vb[0] + h.c0 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot = fmaf(row[q][e], vq[e], dot);
      }
    }
    if (act) sm.part[hh][k + 1 + ii] = dot;
    __syncthreads();
    // K = (tau/2) p.v with p_i = tau (part0_i + part1_i), formed alike by
    // every wave, then w_c = p_c - K v_c into the wave's own copy of w (zero
    // left of the block); the wave reads back only what it wrote itself
    float* wb = sm.wb[tid >> 6];
    {
      const int ca = lane, cb = lane + 64;
      const bool ina = ca >= k + 1, inb = cb >= k + 1 && cb < D;
      const float pa = ina ? pvec(ca, tk) : 0.f, pb = inb ? pvec(cb, tk) : 0.f;
      const float va = ina ? sm.vb[0][ca] : 0.f, vbb = inb ? sm.vb[0][cb] : 0.f;
      const float kc = 0.5f * tk * wave_sum(fmaf(pa, va, pb * vbb));
      wb[ca] = ina ? __fsub_rn(pa, __fmul_rn(kc, va)) : 0.f;
      if (cb < D) wb[cb] = inb ? __fsub_rn(pb, __fmul_rn(kc, vbb)) : 0.f;
    }
    if (act) {
      const int r = k + 1 + ii;
      const float vi = sm.vb[0][r], wi = wb[r];
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        if (q < h.n) {
          const int c = h.c0 + 4 * q;
          const f32x4_t vq = lds4(sm.vb[0] + c), wq = lds4(wb + c);
          // columns left of the block have v = w = 0: they are written back unchanged
          f32x4_t o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __fsub_rn(row[q][e], sym2(vi, wq[e], wi, vq[e]));
          sts4(ar + 4 * q, o);
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    sm.de[0][1][0] = sm.de[1][1][0] = A[(D - 2) * S + D - 2];
    sm.de[0][0] = sm.de[1][0] = f32x2_t{A[(D - 1) * S + D - 1], A[(D - 2) * S + D - 1]};
    sm.de[0][D - 1][1] = sm.de[1][D - 1][1] = 0.f;
  }
  __syncthreads();
}

// Q^T = H_{D-3} ... H_0, accumulated from the last reflector back in place:
// before step k the unit vector fills row and column k+1 of the block
// [k+1.., k+1..]; then Q^T_b -= tau (Q^T_b v) v^T.  Thread (hh, ii) owns
// row k+1+ii of the block over column half hh.  The reflector of step k is
// row k (outside the block), those of later steps were used already.
template <int D>
__device__ __forceinline__ void accumulate_qt(EigSmem<D>& sm, int tid) {
  constexpr int S = EigSmem<D>::S, NC = D / 8;
  float* A = sm.a;
  const int hh = tid >> 7, ii = tid & 127;
  if (tid == 0) A[(D - 1) * S + D - 1] = 1.f;
  for (int k = D - 3; k >= 0; --k) {
    const int m = D - 1 - k;
    for (int c = tid; c < D; c += kEigThreads) {
      sm.vb[0][c] = c < k + 1 ? 0.f : (c == k + 1 ? 1.f : A[k * S + c]);
      if (c >= k + 1) {
        A[(k + 1) * S + c] = c == k + 1 ? 1.f : 0.f;   // row k+1
        A[c * S + k + 1] = c == k + 1 ? 1.f : 0.f;     // column k+1
      }
    }
    __syncthreads();
    const float tk = sm.tau[k];
    if (tk == 0.f) continue;
    const Halves h = half_of<D>(k, hh);
    const bool act = ii < m;
    float* ar = A + (k + 1 + ii) * S + h.c0;
    f32x4_t row[NC];
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      if (q < h.n && act) {
        row[q] = lds4(ar + 4 * q);
        const f32x4_t vq = lds4(sm.vb[0] + h.c0 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot = fmaf(row[q][e], vq[e], dot);
      }
    }
    if (act) sm.part[hh][k + 1 + ii] = dot;
    __syncthreads();
    if (act) {
      const float tw = tk * (sm.part[0][k + 1 + ii] + sm.part[1][k + 1 + ii]);
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        if (q < h.n) {
          const f32x4_t vq = lds4(sm.vb[0] + h.c0 + 4 * q);   // zero left of the block: those entries stay
          f32x4_t o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = fmaf(-tw, vq[e], row[q][e]);
          sts4(ar + 4 * q, o);
        }
      }
    }
    __syncthreads();
  }
  for (int c = tid; c < D; c += kEigThreads) {
    A[c] = c == 0 ? 1.f : 0.f;       // row 0
    A[c * S] = c == 0 ? 1.f : 0.f;   // column 0
  }
  __syncthreads();
}

// Entry i (uniform) of a vector held across the lanes of two registers
// (lane i % 64 of lo for i < 64, of hi otherwise).
template <int D>
__device__ __forceinline__ float lane_get(float lo, float hi, int i) {
  const float v = (D > 64 && i >= 64) ? hi : lo;
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i & 63));
}

// Implicit QL on (d, e) of this wave's copy; rotations applied to entries
// 64 w + lane of the rows of Q^T (one wave per 64 entries).  Returns the
// iteration count, negative when an eigenvalue took more than kEigMaxIt
// iterations.  Every lane computes the same scalar recurrence.  At the start
// of an iteration (d, e) is read from LDS into lane registers for the
// deflation test and the shift; the sweep reads each pair one step ahead
// (before it is changed) and writes the new pair of the step behind it.  A
// rotation of f = g = 0 is the identity (c = 1, s = 0, r = 0), so a sweep
// never stops early.
template <int D>
__device__ __forceinline__ int ql_implicit(EigSmem<D>& sm, int wave, int lane, float tol_abs) {
  constexpr int S = EigSmem<D>::S;
  f32x2_t* de = sm.de[wave];
  // the QL runs on the reversed tridiagonal (it converges in fewer
  // rotations from that end for these graded matrices): its index i is row
  // D-1-i of Q^T, and Q^T[D-1-i][64 w + lane] is at zr[-i * S]
  float* zr = sm.a + (D - 1) * S + 64 * wave + lane;
  int iters = 0;
  for (int l = 0; l < D; ++l) {
    for (int it = 0;; ++it) {
      const f32x2_t plo = de[lane], phi = D > 64 ? de[min(lane + 64, D - 1)] : f32x2_t{0.f, 0.f};
      const float dlo = plo[0], elo = plo[1], dhi = phi[0], ehi = phi[1];
      // m = the first index >= l whose e_m is negligible (e_{D-1} = 0)
      int m = D - 1;
      {
        const float d64 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dhi), 0));
        const float d1lo = lane == 63 ? d64 : __shfl_down(dlo, 1);
        const bool nega = lane >= l && lane < D - 1 &&
                          (fabsf(elo) <= kEigTolRel * (fabsf(dlo) + fabsf(d1lo)) || fabsf(elo) <= tol_abs);
        const uint64_t ba = __builtin_amdgcn_ballot_w64(nega);
        if (ba != 0) {
          m = __builtin_ctzll(ba);
        } else if (D > 64) {
          const float d1hi = __shfl_down(dhi, 1);
          const int jb = lane + 64;
          const bool negb = jb >= l && jb < D - 1 &&
                            (fabsf(ehi) <= kEigTolRel * (fabsf(dhi) + fabsf(d1hi)) || fabsf(ehi) <= tol_abs);
          const uint64_t bb = __builtin_amdgcn_ballot_w64(negb);
          if (bb != 0) m = 64 + __builtin_ctzll(bb);
        }
      }
      if (m == l) break;
      if (it == kEigMaxIt) return -(iters + 1);
      ++iters;
      const float dl = lane_get<D>(dlo, dhi, l), el = lane_get<D>(elo, ehi, l);
      float g = (lane_get<D>(dlo, dhi, l + 1) - dl) / (2.f * el);
      const float rr = sqrtf(fmaf(g, g, 1.f));
      g = lane_get<D>(dlo, dhi, m) - dl + el / (g + copysignf(rr, g));
      float s = 1.f, c = 1.f, p = 0.f;
      float zc = zr[-m * S];
      float dn = lane_get<D>(dlo, dhi, m);   // d_{i+1} before this sweep
      f32x2_t cur = de[m - 1];               // (d_i, e_i) of the step
      for (int i = m - 1; i >= l; --i) {
        const f32x2_t nxt = de[i > 0 ? i - 1 : 0];   // next step's pair (not yet changed)
        const float zi = zr[-i * S];
        const float di = cur[0], ei = cur[1];
        const float f = s * ei, b = c * ei, b2 = 2.f * b;
        const float r2 = fmaf(f, f, g * g);
        // r2 = 0 (f = g = 0): ri is finite, s = 0 and c = 0 + 1
        const float one = r2 == 0.f ? 1.f : 0.f;
        const float ri = __builtin_amdgcn_rsqf(fmaxf(r2, 0x1p-126f));
        s = f * ri;
        c = fmaf(g, ri, one);
        const float gg = dn - p;
        const float t = fmaf(di - gg, s, c * b2);
        p = s * t;
        de[i + 1] = f32x2_t{gg + p, r2 * ri};
        g = fmaf(c, t, -b);
        zr[-(i + 1) * S] = fmaf(s, zi, c * zc);
        zc = fmaf(c, zi, -s * zc);
        dn = di;
        cur = nxt;
      }
      de[l] = f32x2_t{dn - p, g};
      de[m][1] = 0.f;
      zr[-l * S] = zc;
    }
  }
  return iters;
}

template <int D, int DT>
__global__ __launch_bounds__(kEigThreads) void milo_encode_spectrum_kernel(EncodeParams p) {
  __shared__ __attribute__((aligned(16))) EigSmem<D> sm;
  constexpr int S = EigSmem<D>::S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.x;
  const EncMat e = enc_mat(p, m, D);
  const void* x = e.kv ? p.v : p.k;

  if (DT == MILO_BF16)
    gram_bf16<D>(reinterpret_cast<const uint16_t*>(x), e.row0, e.T, sm, tid);
  else
    gram_f32<D>(reinterpret_cast<const float*>(x), e.row0, e.T, sm, tid);
  __syncthreads();
  // exact symmetry from the upper triangle; the trace
  for (int q = tid; q < D * D; q += kEigThreads) {
    const int i = q / D, j = q % D;
    if (i > j) sm.a[i * S + j] = sm.a[j * S + i];
  }
  if (tid < 64) {
    float t = 0.f;
    for (int i = tid; i < D; i += 64) t += sm.a[i * S + i];
    t = wave_sum(t);
    if (tid == 0) sm.trace = t;
  }
  __syncthreads();
  const float trace = sm.trace;
  const bool finite = trace < __builtin_huge_valf();   // false for inf and NaN (inputs must be finite)
  int iters = finite ? 0 : -1;
  float unscale = 0.f;
  if (trace > 0.f && finite) {
    int ex;
    frexpf(trace, &ex);
    for (int q = tid; q < D * D; q += kEigThreads) {
      const int i = q / D, j = q % D;
      sm.a[i * S + j] = ldexpf(sm.a[i * S + j], -ex);   // exact
    }
    unscale = ldexpf(1.f, ex);
    __syncthreads();
    tridiagonalize<D>(sm, tid);
    accumulate_qt<D>(sm, tid);
    if (wave < D / 64) {
      const int it = ql_implicit<D>(sm, wave, lane, kEigTolAbs * ldexpf(trace, -ex));
      if (tid == 0) iters = it;
      if (wave == 0) {   // eigenvalues out (wave 1 works on its own copy)
        sm.lam[D - 1 - lane] = sm.de[0][lane][0];   // by row of Q^T
        if (D > 64) sm.lam[D - 65 - lane] = sm.de[0][lane + 64][0];
      }
    }
  } else {
    // no energy: eigenvalues 0, eigenvectors the unit vectors
    for (int q = tid; q < D * D; q += kEigThreads) {
      const int i = q / D, j = q % D;
      sm.a[i * S + j] = i == j ? 1.f : 0.f;
    }
    for (int i = tid; i < D; i += kEigThreads) sm.lam[i] = 0.f;
  }
  __syncthreads();

  // ---- sort by descending eigenvalue; sigma and eigenvector rows out
  if (tid < D) {
    const float li = sm.lam[tid];
    int r = 0;
    for (int j = 0; j < D; ++j) {
      const float lj = sm.lam[j];
      r += (lj > li) || (lj == li && j < tid);
    }
    sm.rank[tid] = r;
    if (p.sigma) p.sigma[(size_t)m * D + r] = finite ? sqrtf(fmaxf(li * unscale, 0.f)) : __builtin_nanf("");
  }
  __syncthreads();
  float* vec = p.vecs + (size_t)m * D * D;
  for (int q = tid; q < D * D; q += kEigThreads) {
    const int i = q / D, j = q % D;   // eigenvector i (row i of Q^T), component j
    vec[(size_t)sm.rank[i] * D + j] = sm.a[i * S + j];
  }
  if (tid == 0 && p.iters) p.iters[m] = iters;
}

template <int D, int DT>
__global__ __launch_bounds__(kEncThreads) void milo_encode_factors_kernel(EncodeParams p) {
  constexpr int S = D + 1;
  __shared__ __attribute__((aligned(16))) float wl[D * S];            // W rows
  __shared__ __attribute__((aligned(16))) float xl[kFacTokens * S];   // token rows of X
  const int tid = threadIdx.x;
  const int m = blockIdx.x;
  const EncMat e = enc_mat(p, m, D);
  const milo_block blk = p.blocks[e.b];
  const int rk = min(max(blk.rank_k, 0), D), rv = min(max(blk.rank_v, 0), D);
  const int r = e.kv ? rv : rk;
  const int ld = blk.ld_tok;
  if (r == 0) return;
  const int64_t head = blk.off + (int64_t)e.g * (rk + rv) * (ld + D);
  const int64_t u_off = head + (e.kv ? (int64_t)rk * (ld + D) : 0);
  const int64_t w_off = u_off + (int64_t)r * ld;
  const void* x = e.kv ? p.v : p.k;

  // W: the first r eigenvector rows, to LDS (fp32) and to the pool
  const float* vec = p.vecs + (size_t)m * D * D;
  for (int q = tid; q < r * D; q += kEncThreads) {
    const float w = vec[q];
    wl[(q / D) * S + q % D] = w;
    store1<DT>(p.pool, w_off + q, w);
  }

  // U^T[k][t] = sum_j W[k][j] X[t][j]: thread owns ranks k0..k0+3 and
  // tokens t0..t0+3 of each chunk; tokens T..ld-1 are written as zeros
  const int k0 = (tid >> 4) * 4, t0 = (tid & 15) * 4;
  for (int c0 = 0; c0 < ld; c0 += kFacTokens) {
    __syncthreads();   // W is in LDS / the previous chunk's reads are done
    for (int q = tid; q < kFacTokens * (D / 8); q += kEncThreads) {
      const int t = q / (D / 8), c = (q % (D / 8)) * 8;
      float v8[8];
      if (c0 + t < e.T) {
        load8<DT>(x, e.row0 + (int64_t)(c0 + t) * D + c, v8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) xl[t * S + c + i] = v8[i];
    }
    __syncthreads();
    if (k0 < r) {
      float acc[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
      const int kmax = min(4, r - k0);
      for (int j = 0; j < D; ++j) {
        float wa[4], xb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) wa[a] = a < kmax ? wl[(k0 + a) * S + j] : 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) xb[b] = xl[(t0 + b) * S + j];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(wa[a], xb[b], acc[a][b]);
      }
      const int t = c0 + t0;   // ld is a multiple of 8: the four tokens are all inside or all past it
      if (t < ld) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
          if (a < kmax) store4<DT>(p.pool, u_off + (int64_t)(k0 + a) * ld + t, acc[a]);
      }
    }
  }
}


// Factors for bf16 storage on the matrix cores: U^T = W X^T as
// v_mfma_f32_16x16x32_bf16 with W (fp32) split into bf16 hi + lo (about 17
// significant bits; the X products are exact and the sums fp32), stored
// rounded to nearest even.  Workgroup (matrix, c) of kFacGroups per matrix
// takes the 256-token chunks c, c + kFacGroups, ...; its wave w the 16-rank
// tiles w and w + 4.  Lane l of a tile's 16 x 16 result holds token l%16 of
// the step and ranks 4(l/16) .. +3; tokens past n_tok load as zero, so U^T is
// zero up to ld_tok.  The workgroup of chunk 0 also writes W.
constexpr int kFacGroups = 4;
constexpr int kFacChunk = 256;

template <int D>
__global__ __launch_bounds__(256) void milo_encode_factors_mfma_kernel(EncodeParams p) {
  constexpr int KS = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.x / kFacGroups, grp = blockIdx.x % kFacGroups;
  const EncMat e = enc_mat(p, m, D);
  const milo_block blk = p.blocks[e.b];
  const int rk = min(max(blk.rank_k, 0), D), rv = min(max(blk.rank_v, 0), D);
  const int r = e.kv ? rv : rk;
  const int ld = blk.ld_tok;
  if (r == 0) return;
  const int64_t head = blk.off + (int64_t)e.g * (rk + rv) * (ld + D);
  const int64_t u_off = head + (e.kv ? (int64_t)rk * (ld + D) : 0);
  const int64_t w_off = u_off + (int64_t)r * ld;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(e.kv ? p.v : p.k);
  const float* vec = p.vecs + (size_t)m * D * D;
  if (grp == 0)
    for (int q = tid; q < r * D; q += 256) store1<MILO_BF16>(p.pool, w_off + q, vec[q]);
  const int col = lane & 15, quad = lane >> 4;
  for (int kt = wave; 16 * kt < r; kt += 4) {
    // W rows 16 kt + col (clamped; rows past r are not stored), dims 32 s + 8 quad .. +7
    const float* wr = vec + (size_t)min(16 * kt + col, r - 1) * D + 8 * quad;
    u32x4_t ah[KS], al[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) split_pair(ld16f(wr + 32 * s), ld16f(wr + 32 * s + 4), ah[s], al[s]);
    for (int c0 = grp * kFacChunk; c0 < ld; c0 += kFacGroups * kFacChunk) {
      const int c1 = min(c0 + kFacChunk, ld);
      for (int t0 = c0; t0 < c1; t0 += 16) {
        const int t = t0 + col;
        const uint16_t* xr = x + e.row0 + (int64_t)t * D + 8 * quad;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4_t b = t < e.T ? ld16(xr + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
          acc = mfma32(ah[s], b, acc);
          acc = mfma32(al[s], b, acc);
        }
        if (t < c1) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int k = 16 * kt + 4 * quad + v;
            if (k < r) store1<MILO_BF16>(p.pool, u_off + (int64_t)k * ld + t, acc[v]);
          }
        }
      }
    }
  }
}

template <int D, int DT>
hipError_t launch_enc(const EncodeParams& p, bool spectrum, hipStream_t s) {
  const int64_t mats = (int64_t)p.n_blocks * p.n_kv_heads * 2;
  if (mats == 0) return hipSuccess;
  if (spectrum) {
    hipLaunchKernelGGL((milo_encode_spectrum_kernel<D, DT>), dim3((unsigned)mats), dim3(kEigThreads), 0, s, p);
  } else {
    if constexpr (DT == MILO_BF16)
      hipLaunchKernelGGL((milo_encode_factors_mfma_kernel<D>), dim3((unsigned)(mats * kFacGroups)), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((milo_encode_factors_kernel<D, DT>), dim3((unsigned)mats), dim3(kEncThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_enc_any(const EncodeParams& p, int dtype, int head_dim, bool spectrum, hipStream_t s) {
  if (dtype == MILO_BF16 && head_dim == 128) return launch_enc<128, MILO_BF16>(p, spectrum, s);
  if (dtype == MILO_BF16 && head_dim == 64) return launch_enc<64, MILO_BF16>(p, spectrum, s);
  if (dtype == MILO_F32 && head_dim == 128) return launch_enc<128, MILO_F32>(p, spectrum, s);
  if (dtype == MILO_F32 && head_dim == 64) return launch_enc<64, MILO_F32>(p, spectrum, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode_spectrum(const EncodeParams& p, int dtype, int head_dim, hipStream_t s) {
  return launch_enc_any(p, dtype, head_dim, true, s);
}
hipError_t launch_encode_factors(const EncodeParams& p, int dtype, int head_dim, hipStream_t s) {
  return launch_enc_any(p, dtype, head_dim, false, s);
}

}  // namespace milo
