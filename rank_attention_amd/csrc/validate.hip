// validate.hip -- device-side check of the caller-owned tables (descriptors,
// CSR, tail lengths) against the contract in include/milo_attn.h.  Reads
// only the tables, never the pool; records the smallest (rule, index) of
// any violation with a 64-bit atomic minimum.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kValThreads = 256;

__global__ void milo_validate_init_kernel(unsigned long long* status) { *status = ~0ull; }

__device__ __forceinline__ void report(unsigned long long* status, int rule, int64_t index) {
  atomicMin(status, ((unsigned long long)rule << 32) | (unsigned long long)(uint32_t)index);
}

__global__ __launch_bounds__(kValThreads) void milo_validate_kernel(ValidateParams p) {
  const int64_t idx = (int64_t)blockIdx.x * kValThreads + threadIdx.x;
  if (idx < p.n_descriptors) {
    const milo_block blk = p.blocks[idx];
    const int d = p.head_dim;
    if (blk.rank_k < 0 || blk.rank_k > d || blk.rank_v < 0 || blk.rank_v > d) report(p.status, 3, idx);
    const int ld_align = p.q8 ? 63 : 7, off_align = p.q8 ? 15 : 7;
    if (blk.n_tok < 0 || blk.ld_tok < blk.n_tok || (blk.ld_tok & ld_align) != 0) report(p.status, 4, idx);
    if (blk.off < 0 || (blk.off & off_align) != 0) report(p.status, 5, idx);
    const int64_t rk = min(max(blk.rank_k, 0), d), rv = min(max(blk.rank_v, 0), d);
    const int64_t ld = max(blk.ld_tok, 0);
    // elements of the pool's dtype, or bytes of the 8-bit layout
    const int64_t nt = max(blk.n_tok, 0), rk16 = (rk + 15) & ~15ll;
    const int64_t size = p.q8 ? (int64_t)p.n_kv_heads * (nt * rk16 + rv * ld + (rk + rv) * 2 * d +
                                                         ((8 * (rk + rv) + 15) & ~15ll))
                              : (int64_t)p.n_kv_heads * (rk + rv) * (ld + d);
    if (blk.off >= 0 && blk.off + size > p.pool_elems) report(p.status, 6, idx);
  }
  if (idx < p.n_seqs_checked) {
    const int a = p.seq_blocks[idx], b = p.seq_blocks[idx + 1];
    if (a < 0 || b < a || b > p.n_descriptors) report(p.status, 1, idx);
    if ((int64_t)b - a > p.max_blocks) report(p.status, 2, idx);
  }
  if (idx < p.batch && p.tail_cap > 0) {
    const int L = p.tail_len[idx];
    if (L < p.tail_min || L > p.tail_cap) report(p.status, 7, idx);
  }
}

}  // namespace

hipError_t launch_validate(const ValidateParams& p, hipStream_t s) {
  hipLaunchKernelGGL(milo_validate_init_kernel, dim3(1), dim3(1), 0, s, p.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = std::max<int64_t>(std::max<int64_t>(p.n_descriptors, p.n_seqs_checked), std::max(p.batch, 1));
  hipLaunchKernelGGL(milo_validate_kernel, dim3((unsigned)((n + kValThreads - 1) / kValThreads)),
                     dim3(kValThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace milo
