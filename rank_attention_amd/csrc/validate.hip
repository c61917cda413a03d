// validate.hip -- device-side check of the caller-owned tables (descriptors,
// CSR, tail lengths, the decode schedule) against the contract in
// include/milo_attn.h.  Reads only the tables, never the pool; records the
// smallest (rule, index) of any violation with a 64-bit atomic minimum.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kValThreads = 256;

// status word to "no violation"; the schedule's per-unit counts to zero
__global__ __launch_bounds__(kValThreads) void milo_validate_init_kernel(ValidateParams p) {
  const int64_t idx = (int64_t)blockIdx.x * kValThreads + threadIdx.x;
  if (idx == 0) *p.status = ~0ull;
  if (p.unit_order && idx < p.n_units) p.unit_count[idx] = 0;
}

__device__ __forceinline__ void report(unsigned long long* status, int rule, int64_t index) {
  atomicMin(status, ((unsigned long long)rule << 32) | (unsigned long long)(uint32_t)index);
}

__global__ __launch_bounds__(kValThreads) void milo_validate_kernel(ValidateParams p) {
  const int64_t idx = (int64_t)blockIdx.x * kValThreads + threadIdx.x;
  if (idx < p.n_descriptors) {
    const milo_block blk = p.blocks[idx];
    const int d = p.head_dim;
    if (blk.rank_k < 0 || blk.rank_k > d || blk.rank_v < 0 || blk.rank_v > d) report(p.status, 3, idx);
    const bool bytes = p.dtype == MILO_BF16_Q8 || p.dtype == MILO_BF16_KV4 || p.dtype == MILO_BF16_KV2;
    const int ld_align = bytes ? 63 : 7, off_align = bytes ? 15 : 7;
    if (blk.n_tok < 0 || blk.ld_tok < blk.n_tok || (blk.ld_tok & ld_align) != 0) report(p.status, 4, idx);
    if (blk.off < 0 || (blk.off & off_align) != 0) report(p.status, 5, idx);
    const int64_t rk = min(max(blk.rank_k, 0), d), rv = min(max(blk.rank_v, 0), d);
    const int64_t ld = max(blk.ld_tok, 0);
    // elements of the pool's dtype, or bytes of the 8-bit and KIVI-style layouts
    const int64_t nt = max(blk.n_tok, 0), rk16 = (rk + 15) & ~15ll;
    int64_t size = (int64_t)p.n_kv_heads * (rk + rv) * (ld + d);
    if (p.dtype == MILO_BF16_Q8)
      size = (int64_t)p.n_kv_heads * (nt * rk16 + rv * ld + (rk + rv) * 2 * d + ((8 * (rk + rv) + 15) & ~15ll));
    else if (p.dtype == MILO_BF16_KV4 || p.dtype == MILO_BF16_KV2) {
      const int64_t h = kivi_head_bytes(ld / 64, rk, rv, d, p.dtype == MILO_BF16_KV4 ? 4 : 2);
      if (h > (int64_t)0xFFFFFFFFll) report(p.status, 4, idx);   // the kernel's 32-bit table offsets
      size = (int64_t)p.n_kv_heads * h;
    }
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
  if (p.unit_order && idx < p.n_units) {
    const int u = p.unit_order[idx];
    if (u >= 0 && (int64_t)u < p.n_units) atomicAdd(&p.unit_count[u], 1u);
  }
}

// The schedule is a permutation iff every entry is in range and its unit is
// listed once; positions breaking that are reported (the smallest wins, so
// of two entries naming the same unit the first is reported).
__global__ __launch_bounds__(kValThreads) void milo_validate_order_kernel(ValidateParams p) {
  const int64_t idx = (int64_t)blockIdx.x * kValThreads + threadIdx.x;
  if (idx >= p.n_units) return;
  const int u = p.unit_order[idx];
  if (u < 0 || (int64_t)u >= p.n_units || p.unit_count[u] != 1u) report(p.status, 8, idx);
}

}  // namespace

hipError_t launch_validate(const ValidateParams& p, hipStream_t s) {
  const int64_t nu = p.unit_order ? p.n_units : 0;
  const unsigned init_grid = (unsigned)((std::max<int64_t>(nu, 1) + kValThreads - 1) / kValThreads);
  hipLaunchKernelGGL(milo_validate_init_kernel, dim3(init_grid), dim3(kValThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = std::max<int64_t>(std::max<int64_t>(std::max<int64_t>(p.n_descriptors, p.n_seqs_checked),
                                                        std::max(p.batch, 1)), nu);
  hipLaunchKernelGGL(milo_validate_kernel, dim3((unsigned)((n + kValThreads - 1) / kValThreads)),
                     dim3(kValThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || nu == 0) return e;
  hipLaunchKernelGGL(milo_validate_order_kernel, dim3((unsigned)((nu + kValThreads - 1) / kValThreads)),
                     dim3(kValThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace milo
