// rank.hip -- gfx950 entropy-driven rank allocation over block spectra.
//
// MILO (summary at paperlayer.ai/abs/2609.29913v1, "4.3 Dynamic Rank
// Allocation") sets block ranks under a fixed total budget: every block
// starts at a minimum rank and the remaining rank units go greedily to the
// block whose next unit has the largest marginal information gain, which
// favours slowly decaying spectra.  Keys and values get their own budgets
// ("4.4 MILO Workflow").  Readings of what the pages leave open: a block's
// distribution p is its normalised energy sigma_i^2 / sum sigma^2, averaged
// over its KV heads and renormalised; its entropy H = -sum p ln p; the gain
// of the unit that raises rank r to r + u is H * (p_r + ... + p_{r+u-1});
// ties go to the lowest block index.
//
// Because p is non-increasing within a block, so are its unit gains, and
// the greedy's picks are exactly the K largest gains in the order (gain
// descending, block ascending, unit ascending).  The select kernel finds
// them without a sequential loop: the largest threshold tau (a 32-bit
// pattern of the non-negative fp32 gains, searched bit by bit) with
// count(gain >= tau) >= K; every block takes its units above tau, and the
// units equal to tau are handed out in block order by a prefix count.
//
//  gains   one wave per (block, K/V): p, H and the unit gains (fp32, in a
//          fixed order of operations so that the gains stay non-increasing)
//  select  one 1024-thread workgroup per K/V: threshold search and ranks
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kSelThreads = 1024;

__device__ __forceinline__ uint32_t gain_key(float g) { return __float_as_uint(g); }

template <int D>
__global__ __launch_bounds__(64) void milo_rank_gains_kernel(RankParams p) {
  __shared__ float pl[D];
  const int lane = threadIdx.x;
  const int kv = blockIdx.x & 1, b = blockIdx.x >> 1;
  constexpr int PER = (D + 63) / 64;
  float pb[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) pb[j] = 0.f;
  for (int g = 0; g < p.n_kv_heads; ++g) {
    const float* s = p.sigma + (((size_t)b * p.n_kv_heads + g) * 2 + kv) * D;
    float e[PER], tot = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = lane + 64 * j;
      const float x = i < D ? s[i] : 0.f;
      e[j] = __fmul_rn(x, x);
      tot = __fadd_rn(tot, e[j]);
    }
    tot = wave_sum(tot);
    if (tot > 0.f) {
#pragma unroll
      for (int j = 0; j < PER; ++j) pb[j] = __fadd_rn(pb[j], __fdiv_rn(e[j], tot));
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    pb[j] = __fdiv_rn(pb[j], (float)p.n_kv_heads);
    sum = __fadd_rn(sum, pb[j]);
  }
  sum = wave_sum(sum);
  float h = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (sum > 0.f) pb[j] = __fdiv_rn(pb[j], sum);
    if (pb[j] > 0.f) h -= pb[j] * __logf(pb[j]);
    const int i = lane + 64 * j;
    if (i < D) pl[i] = pb[j];
  }
  h = wave_sum(h);
  h = h > 0.f ? h : 0.f;
  if (lane == 0 && p.entropy) p.entropy[(size_t)b * 2 + kv] = h;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // unit j covers components r_min + j*u .. r_min + (j+1)*u - 1, summed in
  // ascending order
  float* gains = p.gains + ((size_t)kv * p.n_blocks + b) * p.n_units;
  for (int j = lane; j < p.n_units; j += 64) {
    float w = 0.f;
    const int i0 = p.r_min + j * p.unit;
    for (int i = i0; i < i0 + p.unit; ++i) w = __fadd_rn(w, pl[i]);
    const float gval = __fmul_rn(h, w);
    gains[j] = gval > 0.f ? gval : 0.f;   // +0 for zero and -0 alike
  }
}

// Units of block b (gains non-increasing) whose key is >= c: binary search.
__device__ __forceinline__ int count_ge(const float* g, int n, uint32_t c) {
  int lo = 0, hi = n;   // g[0..lo) >= c, g[hi..n) < c
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (gain_key(g[mid]) >= c) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int64_t block_reduce_sum(int64_t v, int64_t* red, int tid) {
  // wave partial sums through LDS, then one thread adds the 16 waves
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();                       // previous use of red is finished
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  int64_t s = 0;
  for (int w = 0; w < kSelThreads / 64; ++w) s += red[w];
  return s;
}

__global__ __launch_bounds__(kSelThreads) void milo_rank_select_kernel(RankParams p) {
  __shared__ int64_t red[kSelThreads / 64];
  __shared__ int scan[kSelThreads];
  const int tid = threadIdx.x;
  const int kv = blockIdx.x;
  const int nb = p.n_blocks, nu = p.n_units;
  const int64_t K = kv ? p.k_units_v : p.k_units_k;
  const float* gains = p.gains + (size_t)kv * nb * nu;

  // largest tau with count(key >= tau) >= K (K >= 1; every key >= 0 counts)
  uint32_t tau = 0;
  if (K > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int64_t c = 0;
      for (int b = tid; b < nb; b += kSelThreads) c += count_ge(gains + (size_t)b * nu, nu, cand);
      if (block_reduce_sum(c, red, tid) >= K) tau = cand;
    }
  }

  // ranks: units above tau, then ties in block order
  int64_t need = 0;
  if (K > 0) {
    int64_t c = 0;
    for (int b = tid; b < nb; b += kSelThreads) c += count_ge(gains + (size_t)b * nu, nu, tau + 1u);
    need = K - block_reduce_sum(c, red, tid);
  }
  int64_t carry = 0;
  for (int base = 0; base < nb; base += kSelThreads) {
    const int b = base + tid;
    int gt = 0, eq = 0;
    if (b < nb && K > 0) {
      const float* g = gains + (size_t)b * nu;
      gt = count_ge(g, nu, tau + 1u);
      eq = count_ge(g, nu, tau) - gt;
    }
    // inclusive scan of eq over this chunk (Hillis-Steele in LDS)
    __syncthreads();
    scan[tid] = eq;
    __syncthreads();
    for (int off = 1; off < kSelThreads; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int64_t before = carry + scan[tid] - eq;   // ties of earlier blocks
    int64_t take = need - before;
    take = take < 0 ? 0 : (take > eq ? eq : take);
    if (b < nb) p.ranks[(size_t)b * 2 + kv] = p.r_min + p.unit * (int32_t)(gt + take);
    carry += scan[kSelThreads - 1];
  }
}

}  // namespace

hipError_t launch_rank(const RankParams& p, int head_dim, hipStream_t s) {
  if (p.n_blocks == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(milo_rank_gains_kernel<128>, dim3((unsigned)(2 * p.n_blocks)), dim3(64), 0, s, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(milo_rank_gains_kernel<64>, dim3((unsigned)(2 * p.n_blocks)), dim3(64), 0, s, p);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(milo_rank_select_kernel, dim3(2), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace milo
