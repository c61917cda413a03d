// merge.hip -- split-K combination of per-unit attention partials (gfx950).
//
// Every work unit of the attention kernels leaves, for each of its query
// rows, the unnormalised output o~_u = sum_t 2^(s_t - m_u) v_t, its running
// max m_u and its sum l_u = sum_t 2^(s_t - m_u) (scores s in log2 units).
// The softmax over the union of the units' tokens is then
//   M = max_u m_u,  l = sum_u l_u 2^(m_u - M),  out = sum_u o~_u 2^(m_u - M) / l,
//   lse = (M + log2 l) ln 2.
// One wave per query row walks the row's units with that running rescale.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

constexpr int kSlotChunk = 256;

template <int D>
__global__ __launch_bounds__(64) void milo_merge_kernel(MergeParams p) {
  constexpr int JPL = D / 64;
  __shared__ float wsh[kSlotChunk];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // (i * q_len + j) * n_q_heads + h
  const int h = row % p.n_q_heads;
  const int ij = row / p.n_q_heads;
  const int j = ij % p.q_len, i = ij / p.q_len;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int g = h / G, hl = h - g * G;
  const int nb = min(max(p.seq_blocks[i + 1] - p.seq_blocks[i], 0), p.max_blocks);
  const size_t rec0 = (size_t)(i * p.n_kv_heads + g) * p.slots * p.rows_per_unit + j * G + hl;
  const size_t rstride = p.rows_per_unit;

  // pass 1: global max over the valid slots (lanes stride over slots)
  float M = kNegInf;
  for (int s = lane; s < p.slots; s += 64) {
    const bool valid = (s == p.tail_slot) || (s < nb);
    if (valid) {
      const size_t rec = rec0 + (size_t)s * rstride;
      const float lu = p.part.ml[rec * 2 + 1];
      if (lu > 0.f) M = fmaxf(M, p.part.ml[rec * 2 + 0]);
    }
  }
  M = wave_max(M);

  // pass 2: weights 2^(m_u - M) per slot through LDS, then o = sum w_u o~_u
  float l = 0.f, o[JPL];
#pragma unroll
  for (int jj = 0; jj < JPL; ++jj) o[jj] = 0.f;
  for (int c0 = 0; c0 < p.slots; c0 += kSlotChunk) {
    const int n = min(kSlotChunk, p.slots - c0);
    for (int k = lane; k < n; k += 64) {
      const int s = c0 + k;
      float w = 0.f;
      if ((s == p.tail_slot) || (s < nb)) {
        const size_t rec = rec0 + (size_t)s * rstride;
        const float lu = p.part.ml[rec * 2 + 1];
        if (lu > 0.f) {
          w = fast_exp2(p.part.ml[rec * 2 + 0] - M);
          l += lu * w;
        }
      }
      wsh[k] = w;
    }
    __syncthreads();
    for (int k0 = 0; k0 < n; k0 += 8) {
      float ov[8][JPL];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = min(k0 + u, n - 1);
        const float* ou = p.part.o + (rec0 + (size_t)(c0 + k) * rstride) * D + lane * JPL;
        const bool take = (k0 + u < n) && wsh[k] > 0.f;
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) ov[u][jj] = take ? ou[jj] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = (k0 + u < n) ? wsh[min(k0 + u, n - 1)] : 0.f;
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) o[jj] = fmaf(w, ov[u][jj], o[jj]);
      }
    }
    __syncthreads();
  }
  l = wave_sum(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = p.out + (size_t)row * D + lane * JPL;
#pragma unroll
  for (int jj = 0; jj < JPL; ++jj) op[jj] = o[jj] * inv;
  if (p.lse && lane == 0) p.lse[row] = l > 0.f ? (M + __log2f(l)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.q_len * p.n_q_heads;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(64);
  if (head_dim == 128)
    hipLaunchKernelGGL(milo_merge_kernel<128>, grid, block, 0, s, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(milo_merge_kernel<64>, grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace milo
