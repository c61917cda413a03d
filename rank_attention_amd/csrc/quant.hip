// quant.hip -- gfx950 8-bit quantisation of a bf16 factor pool.
//
// MILO's cache combines with asymmetric INT8 quantisation (summary at
// paperlayer.ai/abs/2609.29913v1, "5.3 Performance Analysis").  Here the
// token factors carry it: every row of U^T and U'^T (one rank component
// over the block's tokens) gets lo = min, a = (hi - lo) / 255, b = lo and
// codes round_half_even((x - lo) / a) clamped to [0, 255] (0 when a = 0),
// all in correctly rounded fp32, so the codes are a function of the bf16
// inputs alone.  W and W' are copied.  The output is the 8-bit pool layout
// of milo_attn.h.
//
// One 256-thread workgroup per (block, KV head): wave w takes rows w, w+4,
// ... of the head's rank_k + rank_v token-factor rows (min and max are wave
// reductions) and writes the value rows' codes (rank-major in 64-token
// tiles), four per lane and step; then the workgroup writes the key codes
// token-major, one dword of four ranks per thread.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kQuantThreads = 256;

// code of x in a row with minimum lo and step a: round_half_even((x - lo) / a)
// clamped to [0, 255], every step correctly rounded; 0 when a = 0
__device__ __forceinline__ uint32_t quant_code(float x, float lo, float a) {
  if (!(a > 0.f)) return 0u;
  const float q = rintf(__fdiv_rn(__fsub_rn(x, lo), a));
  return (uint32_t)fminf(fmaxf(q, 0.f), 255.f);
}

template <int D>
__global__ __launch_bounds__(kQuantThreads) void milo_quantize_kernel(QuantParams p) {
  __shared__ float lo_s[D], a_s[D];   // the key rows' lo and a
  const int b = blockIdx.x / p.n_kv_heads, g = blockIdx.x % p.n_kv_heads;
  const milo_block sb = p.src_blocks[b], db = p.dst_blocks[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = max(sb.n_tok, 0);
  const int r = min(max(sb.rank_k, 0), D), rv = min(max(sb.rank_v, 0), D);
  const int rk16 = (r + 15) & ~15;
  const int lds = sb.ld_tok, ldd = db.ld_tok;
  const uint16_t* sh = p.src_pool + sb.off + (int64_t)g * (r + rv) * (lds + D);
  const uint16_t* sW = sh + (size_t)r * lds;
  const uint16_t* sUp = sW + (size_t)r * D;
  const uint16_t* sWp = sUp + (size_t)rv * lds;
  uint8_t* dh = p.dst_pool + db.off +
                (int64_t)g * ((int64_t)T * rk16 + (int64_t)rv * ldd + 2 * (int64_t)(r + rv) * D + ((8 * (r + rv) + 15) & ~15));
  uint16_t* dW = reinterpret_cast<uint16_t*>(dh + (int64_t)T * rk16);
  uint8_t* dUp = reinterpret_cast<uint8_t*>(dW + (size_t)r * D);
  uint16_t* dWp = reinterpret_cast<uint16_t*>(dUp + (size_t)rv * ldd);
  float* dsb = reinterpret_cast<float*>(dWp + (size_t)rv * D);

  // every row's lo and a; the value rows' codes (rank-major) at once
  for (int row = wave; row < r + rv; row += kQuantThreads / 64) {
    const uint16_t* src = row < r ? sh + (size_t)row * lds : sUp + (size_t)(row - r) * lds;
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    for (int t = lane; t < T; t += 64) {
      const float x = __uint_as_float((uint32_t)src[t] << 16);
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    float a = 0.f, bias = 0.f;
    if (T > 0) {
      a = __fdiv_rn(__fsub_rn(hi, lo), 255.f);
      bias = lo;
    }
    if (row < r) {
      if (lane == 0) { lo_s[row] = lo; a_s[row] = a; }
    } else {
      // tiles of 64 tokens: token t of value row k at 64 (rv (t / 64) + k) + t % 64
      uint8_t* dst = dUp + (size_t)(row - r) * 64;
      for (int t0 = lane * 4; t0 < ldd; t0 += 256) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + e < T) word |= quant_code(__uint_as_float((uint32_t)src[t0 + e] << 16), lo, a) << (8 * e);
        *reinterpret_cast<uint32_t*>(dst + (size_t)(t0 >> 6) * rv * 64 + (t0 & 63)) = word;
      }
    }
    if (lane == 0) {
      dsb[2 * row] = a;
      dsb[2 * row + 1] = bias;
    }
  }
  // padding of the (a, b) region to 16 bytes
  if ((r + rv) & 1) {
    if (tid < 2) dsb[2 * (r + rv) + tid] = 0.f;
  }
  __syncthreads();
  // key codes token-major: thread per (token, 4 ranks); ranks r .. rk16-1 are 0
  const int wpt = rk16 / 4;
  for (int x = tid; x < T * wpt; x += kQuantThreads) {
    const int t = x / wpt, k0 = 4 * (x - t * wpt);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = k0 + e;
      if (k < r) word |= quant_code(__uint_as_float((uint32_t)sh[(size_t)k * lds + t] << 16), lo_s[k], a_s[k]) << (8 * e);
    }
    *reinterpret_cast<uint32_t*>(dh + (size_t)t * rk16 + k0) = word;
  }
  for (int x = tid; x < r * D; x += kQuantThreads) dW[x] = sW[x];
  for (int x = tid; x < rv * D; x += kQuantThreads) dWp[x] = sWp[x];
}

}  // namespace

hipError_t launch_quantize(const QuantParams& p, int head_dim, hipStream_t s) {
  const int64_t wgs = (int64_t)p.n_blocks * p.n_kv_heads;
  if (wgs == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(milo_quantize_kernel<128>, dim3((unsigned)wgs), dim3(kQuantThreads), 0, s, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(milo_quantize_kernel<64>, dim3((unsigned)wgs), dim3(kQuantThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace milo
