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

template <int D>
__global__ __launch_bounds__(64) void milo_merge_kernel(MergeParams p) {
  constexpr int JPL = D / 64;
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // (i * q_len + j) * n_q_heads + h
  const int h = row % p.n_q_heads;
  const int ij = row / p.n_q_heads;
  const int j = ij % p.q_len, i = ij / p.q_len;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int g = h / G, hl = h - g * G;
  const int nb = min(max(p.seq_blocks[i + 1] - p.seq_blocks[i], 0), p.max_blocks);
  const int r_in = j * G + hl;
  float M = kNegInf, l = 0.f, o[JPL];
#pragma unroll
  for (int jj = 0; jj < JPL; ++jj) o[jj] = 0.f;
  for (int s = 0; s < p.slots; ++s) {
    const bool valid = (s == p.tail_slot) || (s < nb);
    if (!valid) continue;
    const size_t rec = ((size_t)(i * p.n_kv_heads + g) * p.slots + s) * p.rows_per_unit + r_in;
    const float mu = p.part.ml[rec * 2 + 0];
    const float lu = p.part.ml[rec * 2 + 1];
    if (!(lu > 0.f)) continue;
    const float mn = fmaxf(M, mu);
    const float a = fast_exp2(M - mn), b = fast_exp2(mu - mn);
    const float* ou = p.part.o + rec * D + lane * JPL;
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) o[jj] = o[jj] * a + ou[jj] * b;
    l = l * a + lu * b;
    M = mn;
  }
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
