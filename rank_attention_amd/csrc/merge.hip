// merge.hip -- split-K combination of per-unit attention partials (gfx950).
//
// Every work unit of the attention kernels leaves, for each of its query
// rows, the unnormalised output o~_u = sum_t 2^(s_t - m_u) v_t, its running
// max m_u and its sum l_u = sum_t 2^(s_t - m_u) (scores s in log2 units).
// The softmax over the union of the units' tokens is then
//   M = max_u m_u,  l = sum_u l_u 2^(m_u - M),  out = sum_u o~_u 2^(m_u - M) / l,
//   lse = (M + log2 l) ln 2.
// Each query row is folded by one to eight waves with that running rescale.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

constexpr int kMergeBatch = 9;   // slots whose loads one wave issues together

// One workgroup of W waves per query row.  Wave w folds the slots s = w,
// w+W, ... into a running (M, l, o) in batches of nine slots, all of whose
// loads are issued before any is used; the waves' results are then combined
// through LDS.  The launcher picks the fewest waves that cover the slots in
// one batch each (at most eight), so every load of a row is in flight at once
// for up to 72 slots and no wave of a short row idles.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void milo_merge_kernel(MergeParams p) {
  constexpr int kMergeWaves = W;
  constexpr int JPL = D / 64;
  __shared__ float sh_m[kMergeWaves], sh_l[kMergeWaves];
  __shared__ __attribute__((aligned(16))) float sh_o[kMergeWaves][D];   // unused when W = 1
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x;  // (i * q_len + j) * n_q_heads + h
  const int h = row % p.n_q_heads;
  const int ij = row / p.n_q_heads;
  const int j = ij % p.q_len, i = ij / p.q_len;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int g = h / G, hl = h - g * G;
  const int si = i * p.seq_stride;
  const int nb = min(max(p.seq_blocks[si + 1] - p.seq_blocks[si], 0), p.max_blocks);
  const size_t rec0 = (size_t)(i * p.n_kv_heads + g) * p.slots * p.rows_per_unit + j * G + hl;
  const size_t rstride = p.rows_per_unit;

  float M = kNegInf, l = 0.f, o[JPL];
#pragma unroll
  for (int jj = 0; jj < JPL; ++jj) o[jj] = 0.f;
  for (int s0 = wave; s0 < p.slots; s0 += kMergeWaves * kMergeBatch) {
    float mu[kMergeBatch], lu[kMergeBatch], ou[kMergeBatch][JPL];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + u * kMergeWaves;
      const bool valid = s < p.slots && ((s >= p.tail_slot) || s * p.blocks_per_slot < nb);
      const size_t rec = rec0 + (size_t)(valid ? s : 0) * rstride;
      mu[u] = valid ? p.part.ml[rec * 2 + 0] : kNegInf;
      lu[u] = valid ? p.part.ml[rec * 2 + 1] : 0.f;
#pragma unroll
      for (int jj = 0; jj < JPL; ++jj) ou[u][jj] = valid ? p.part.o[rec * D + lane * JPL + jj] : 0.f;
    }
    float bm = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (lu[u] > 0.f) bm = fmaxf(bm, mu[u]);
    if (bm == kNegInf) continue;   // nothing valid yet
    const float a = fast_exp2(M - bm);
    l *= a;
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) o[jj] *= a;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float w = lu[u] > 0.f ? fast_exp2(mu[u] - bm) : 0.f;
      l += lu[u] * w;
#pragma unroll
      for (int jj = 0; jj < JPL; ++jj) o[jj] = fmaf(w, ou[u][jj], o[jj]);
    }
    M = bm;
  }
  // every lane holds the same M and l; one wave needs no combination
  float Mt = M, lt = l, ot[JPL];
#pragma unroll
  for (int jj = 0; jj < JPL; ++jj) ot[jj] = o[jj];
  if constexpr (kMergeWaves > 1) {
    if (lane == 0) { sh_m[wave] = M; sh_l[wave] = l; }
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) sh_o[wave][lane * JPL + jj] = o[jj];
    __syncthreads();
    if (wave != 0) return;
    Mt = kNegInf;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) Mt = fmaxf(Mt, sh_m[w]);
    lt = 0.f;
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) ot[jj] = 0.f;
    if (Mt != kNegInf) {
#pragma unroll
      for (int w = 0; w < kMergeWaves; ++w) {
        const float sc = fast_exp2(sh_m[w] - Mt);
        lt += sh_l[w] * sc;
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) ot[jj] = fmaf(sc, sh_o[w][lane * JPL + jj], ot[jj]);
      }
    }
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float* op = p.out + (size_t)row * D + lane * JPL;
#pragma unroll
  for (int jj = 0; jj < JPL; ++jj) op[jj] = ot[jj] * inv;
  if (p.lse && lane == 0) p.lse[row] = lt > 0.f ? (Mt + __log2f(lt)) * kLn2 : kNegInf;
}

template <int D>
void launch_merge_d(const MergeParams& p, int64_t rows, hipStream_t s) {
  const int need = (p.slots + kMergeBatch - 1) / kMergeBatch;
  const dim3 grid((unsigned)rows);
  if (need <= 1)
    hipLaunchKernelGGL((milo_merge_kernel<D, 1>), grid, dim3(64), 0, s, p);
  else if (need <= 2)
    hipLaunchKernelGGL((milo_merge_kernel<D, 2>), grid, dim3(128), 0, s, p);
  else if (need <= 4)
    hipLaunchKernelGGL((milo_merge_kernel<D, 4>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((milo_merge_kernel<D, 8>), grid, dim3(512), 0, s, p);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.q_len * p.n_q_heads;
  if (rows == 0) return hipSuccess;
  if (head_dim == 128)
    launch_merge_d<128>(p, rows, s);
  else if (head_dim == 64)
    launch_merge_d<64>(p, rows, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace milo
