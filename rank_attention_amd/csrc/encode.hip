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
//  spectrum  G = X^T X in fp32 (products of bf16/fp32 inputs are exact, sums
//            fp32), then the cyclic Jacobi eigenvalue method on G in LDS:
//            every round applies d/2 disjoint plane rotations chosen by the
//            round-robin (circle) pairing, so a sweep of d-1 rounds meets
//            every index pair once.  A rotation's 2x2 blocks of G are
//            owned by single threads, so a round is two barriers; each
//            thread reads all of its blocks before writing any.  Sweeps
//            stop after one without rotations.  Output: sigma_i =
//            sqrt(max(lambda_i, 0)) descending and the eigenvectors as
//            rows, sorted the same way (workspace).
//  factors   W = the first r eigenvector rows, U^T = W X^T (fp32 sums),
//            written into the pool in the storage type (RNE for bf16),
//            U^T rows zero-padded to ld_tok.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kEncThreads = 512;
constexpr int kEncMaxSweeps = 16;
// A rotation is applied when |g_pq| exceeds both tolerances: relative to
// sqrt(|g_pp g_qq|) and absolute relative to trace(G).  Without the absolute
// floor, rounding noise between the tiny eigenvalues of a rank-deficient
// block keeps rotations going in every sweep.
constexpr float kEncTolRel = 1e-7f;
constexpr float kEncTolAbs = 1e-8f;
constexpr int kFacTokens = 64;     // tokens per staged chunk in the factors kernel

template <int D>
struct EncSmem {
  static constexpr int S = D + 1;  // padded row stride
  float g[D * S];
  float v[D * S];                  // eigenvectors (columns); the Gram's staging buffer first
  float pc[D / 2], ps[D / 2], pt[D / 2];
  int pp[D / 2], pq[D / 2];
  int rank[D];
  float trace;
  int nrot;              // rotations in the current sweep
  int nrot_round[2];     // rotations in the current round (alternating by round parity)
};

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

template <int D, int DT>
__global__ __launch_bounds__(kEncThreads) void milo_encode_spectrum_kernel(EncodeParams p) {
  __shared__ __attribute__((aligned(16))) EncSmem<D> sm;
  constexpr int S = EncSmem<D>::S;
  constexpr int H = D / 2;
  constexpr int KS = kEncThreads / H;   // rows of blocks (and of V) between a thread's items
  constexpr int NB = H * H / kEncThreads;   // 2x2 blocks of G per thread per round
  constexpr int NV = D * H / kEncThreads;   // (row, pair) items of V per thread per round
  static_assert(kEncThreads % H == 0 && NB * kEncThreads == H * H && NV * kEncThreads == D * H, "work split");
  const int tid = threadIdx.x;
  const int m = blockIdx.x;
  const EncMat e = enc_mat(p, m, D);
  const void* x = e.kv ? p.v : p.k;

  // ---- G = X^T X: thread owns rows i0..i0+TI-1, columns j0..j0+TJ-1
  constexpr int TI = D / 32, TJ = D / 16;
  const int i0 = (tid >> 4) * TI, j0 = (tid & 15) * TJ;
  float acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = 0.f;
  float* xs = sm.v;   // staging: D token rows x D, row stride D
  for (int t0 = 0; t0 < e.T; t0 += D) {
    const int n = min(D, e.T - t0);
    __syncthreads();   // the previous chunk's reads are done
    for (int q = tid; q < D * (D / 8); q += kEncThreads) {
      const int t = q / (D / 8), c = (q % (D / 8)) * 8;
      float v8[8];
      if (t < n) {
        load8<DT>(x, e.row0 + (int64_t)(t0 + t) * D + c, v8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[t * D + c + i] = v8[i];
    }
    __syncthreads();
    for (int t = 0; t < n; ++t) {
      float a[TI], c[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) a[i] = xs[t * D + i0 + i];
#pragma unroll
      for (int j = 0; j < TJ; ++j) c[j] = xs[t * D + j0 + j];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = fmaf(a[i], c[j], acc[i][j]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) sm.g[(i0 + i) * S + j0 + j] = acc[i][j];
  for (int q = tid; q < D * D; q += kEncThreads) {
    const int i = q / D, j = q % D;
    sm.v[i * S + j] = (i == j) ? 1.f : 0.f;
  }
  if (tid == 0) {
    sm.nrot = 0;
    sm.nrot_round[0] = sm.nrot_round[1] = 0;
  }
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
    for (int i = tid; i < D; i += 64) s += sm.g[i * S + i];
    s = wave_sum(s);
    if (tid == 0) sm.trace = s;
  }
  __syncthreads();
  const float tol_abs = kEncTolAbs * fabsf(sm.trace);

  // ---- cyclic Jacobi sweeps
  int sweeps = 0, rounds = 0;   // rounds: over all sweeps (parity of the round counter)
  bool converged = false;
  while (sweeps < kEncMaxSweeps) {
    ++sweeps;
    for (int rnd = 0; rnd < D - 1; ++rnd, ++rounds) {
      __syncthreads();   // the previous round's updates are visible
      // the previous round's counter was read before the barrier above; it
      // is the one the next round uses, so clear it now
      if (tid == 0) sm.nrot_round[(rounds + 1) & 1] = 0;
      if (tid < H) {
        // circle pairing: position 0 holds index 0, position k > 0 holds
        // 1 + (k - 1 + rnd) mod (D - 1); pair = positions (tid, D - 1 - tid)
        const int ka = tid, kb = D - 1 - tid;
        const int ia = ka == 0 ? 0 : 1 + (ka - 1 + rnd) % (D - 1);
        const int ib = 1 + (kb - 1 + rnd) % (D - 1);
        const int pi = min(ia, ib), qi = max(ia, ib);
        const float gpp = sm.g[pi * S + pi], gqq = sm.g[qi * S + qi], gpq = sm.g[pi * S + qi];
        float c = 1.f, s = 0.f, t = 0.f;
        if (fabsf(gpq) > fmaxf(kEncTolRel * sqrtf(fabsf(gpp * gqq)), tol_abs)) {
          // the smaller-angle root of t^2 + 2 theta t - 1 = 0 zeroes g_pq
          const float theta = (gqq - gpp) / (2.f * gpq);
          t = (theta >= 0.f ? 1.f : -1.f) / (fabsf(theta) + sqrtf(fmaf(theta, theta, 1.f)));
          c = 1.f / sqrtf(fmaf(t, t, 1.f));
          s = t * c;
          atomicAdd(&sm.nrot, 1);
          atomicAdd(&sm.nrot_round[rounds & 1], 1);
        }
        sm.pp[tid] = pi;
        sm.pq[tid] = qi;
        sm.pc[tid] = c;
        sm.ps[tid] = s;
        sm.pt[tid] = t;
      }
      __syncthreads();
      if (sm.nrot_round[rounds & 1] == 0) continue;   // no rotation in this round (uniform)
      // G <- J^T G J, J = the round's rotations ([[c, s], [-s, c]] on (p, q)):
      // 2x2 block (k, l) of G becomes R_k^T B R_l.  Thread tid owns the
      // blocks l = tid % H, k = tid / H + KS * i: it reads all of them, then
      // rotates, then writes (the blocks are disjoint, and an identity
      // rotation reproduces its block exactly, so no block is skipped).
      {
        const int l = tid % H, kb = tid / H;
        const int pl = sm.pp[l], ql = sm.pq[l];
        const float cl = sm.pc[l], sl = sm.ps[l];
        float b[NB][4];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int k = kb + KS * i;
          const int pk = sm.pp[k], qk = sm.pq[k];
          b[i][0] = sm.g[pk * S + pl];
          b[i][1] = sm.g[pk * S + ql];
          b[i][2] = sm.g[qk * S + pl];
          b[i][3] = sm.g[qk * S + ql];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int k = kb + KS * i;
          const int pk = sm.pp[k], qk = sm.pq[k];
          if (k == l) {
            // diagonal block: closed form, a rotated coupling becomes exactly 0
            const float t = sm.pt[k];
            const bool rot = sl != 0.f;
            sm.g[pk * S + pk] = b[i][0] - t * b[i][1];
            sm.g[qk * S + qk] = b[i][3] + t * b[i][1];
            sm.g[pk * S + qk] = rot ? 0.f : b[i][1];
            sm.g[qk * S + pk] = rot ? 0.f : b[i][2];
          } else {
            const float ck = sm.pc[k], sk = sm.ps[k];
            const float m00 = ck * b[i][0] - sk * b[i][2], m01 = ck * b[i][1] - sk * b[i][3];
            const float m10 = sk * b[i][0] + ck * b[i][2], m11 = sk * b[i][1] + ck * b[i][3];
            sm.g[pk * S + pl] = cl * m00 - sl * m01;
            sm.g[pk * S + ql] = sl * m00 + cl * m01;
            sm.g[qk * S + pl] = cl * m10 - sl * m11;
            sm.g[qk * S + ql] = sl * m10 + cl * m11;
          }
        }
        // V <- V J: columns p_l, q_l of rows tid / H + KS * i
        if (sl != 0.f) {
          float va[NV], vb[NV];
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            const int row = kb + KS * i;
            va[i] = sm.v[row * S + pl];
            vb[i] = sm.v[row * S + ql];
          }
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            const int row = kb + KS * i;
            sm.v[row * S + pl] = cl * va[i] - sl * vb[i];
            sm.v[row * S + ql] = sl * va[i] + cl * vb[i];
          }
        }
      }
    }
    __syncthreads();
    const int n = sm.nrot;
    __syncthreads();   // every thread has read the count before it is reset
    if (tid == 0) sm.nrot = 0;
    if (n == 0) {
      converged = true;
      break;
    }
  }

  // ---- sort by descending eigenvalue; sigma and eigenvector rows out
  __syncthreads();
  if (tid < D) {
    const float li = sm.g[tid * S + tid];
    int r = 0;
    for (int j = 0; j < D; ++j) {
      const float lj = sm.g[j * S + j];
      r += (lj > li) || (lj == li && j < tid);
    }
    sm.rank[tid] = r;
    if (p.sigma) p.sigma[(size_t)m * D + r] = sqrtf(fmaxf(li, 0.f));
  }
  __syncthreads();
  float* vec = p.vecs + (size_t)m * D * D;
  for (int q = tid; q < D * D; q += kEncThreads) {
    const int i = q / D, j = q % D;   // eigenvector i (column i of V), component j
    vec[(size_t)sm.rank[i] * D + j] = sm.v[j * S + i];
  }
  if (tid == 0 && p.sweeps) p.sweeps[m] = converged ? sweeps : -sweeps;
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

template <int D, int DT>
hipError_t launch_enc(const EncodeParams& p, bool spectrum, hipStream_t s) {
  const int64_t mats = (int64_t)p.n_blocks * p.n_kv_heads * 2;
  if (mats == 0) return hipSuccess;
  if (spectrum)
    hipLaunchKernelGGL((milo_encode_spectrum_kernel<D, DT>), dim3((unsigned)mats), dim3(kEncThreads), 0, s, p);
  else
    hipLaunchKernelGGL((milo_encode_factors_kernel<D, DT>), dim3((unsigned)mats), dim3(kEncThreads), 0, s, p);
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
