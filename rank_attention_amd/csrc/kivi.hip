// kivi.hip -- gfx950 KIVI-style 4-/2-bit quantisation of a bf16 factor pool.
//
// MILO's cache combines with KIVI quantisation (summary at
// paperlayer.ai/abs/2609.29913v1, "5.3 Performance Analysis"): keys grouped
// per channel, values per token, asymmetric low-bit codes with an fp16 scale
// and bias per group.  Here the token factors carry it: a key group is one
// rank component of U over a 64-token chunk of the block, a value group one
// token of U' over 32 rank components.  Per group of bf16 elements x (in
// fp32), with L = 2^bits - 1:
//     a = fp16((max x - min x) / L),  b = fp16(min x),
//     code = clamp(round_half_even((x - b) / a), 0, L)   (0 when a = 0),
// every fp32 step correctly rounded and a, b taken at their fp16 values, so
// the codes are a function of the bf16 inputs alone.  W and W' are copied.
// The output is the KIVI-style pool layout of milo_attn.h.
//
// One 256-thread workgroup per (block, KV head), looping over the chunks:
//   keys:   wave w takes rank components w, w + 4, ...; lane t holds chunk
//           token t, so a group's min and max are wave reductions;
//   values: thread (token t, group v) reduces its own 32 components;
// the codes of the chunk are staged in LDS ([rank][token] bytes) and then
// packed into the code words of the layout, one word per thread.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr int kKivThreads = 256;

__device__ __forceinline__ uint32_t kiv_code(float x, float b, float a, float L) {
  if (!(a > 0.f)) return 0u;
  const float q = rintf(__fdiv_rn(__fsub_rn(x, b), a));
  return (uint32_t)fminf(fmaxf(q, 0.f), L);
}

__device__ __forceinline__ float bf16_at(const uint16_t* p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

__device__ __forceinline__ uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// Bit position of code i (0..7) of 8-code word `word` (the layout of
// milo_attn.h): 4-bit, nibble 2i (i < 4) or 2(i - 4) + 1; 2-bit (two words
// per dword), pair P = 4 word + i / 2 is in bytes 2 (P % 2) and 2 (P % 2) + 1
// at field P / 2, so code i is at bit 8 (2 (P % 2) + i % 2) + 2 (P / 2).
template <int BITS>
__device__ __forceinline__ int code_shift(int word, int i) {
  if (BITS == 4) return 4 * (i < 4 ? 2 * i : 2 * (i - 4) + 1);
  const int P = 4 * word + i / 2;
  return 8 * (2 * (P % 2) + i % 2) + 2 * (P / 2);
}

template <int D, int BITS>
__global__ __launch_bounds__(kKivThreads) void milo_kivi_quantize_kernel(QuantParams p) {
  constexpr float L = (float)((1 << BITS) - 1);
  __shared__ uint8_t kc[D][64];   // key codes of the chunk, [rank][token]
  __shared__ uint8_t vc[D][64];   // value codes, [rank][token]
  __shared__ float red[2][kKivThreads / 64];
  const int b = blockIdx.x / p.n_kv_heads, g = blockIdx.x % p.n_kv_heads;
  const milo_block sb = p.src_blocks[b], db = p.dst_blocks[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = max(sb.n_tok, 0);
  const int r = min(max(sb.rank_k, 0), D), rv = min(max(sb.rank_v, 0), D);
  const int nch = max(db.ld_tok, 0) / 64;
  const int ng8 = (r + 7) / 8, ngv = (rv + 31) / 32, ntv = (rv + 15) / 16;
  const int lds = sb.ld_tok;
  const uint16_t* sh = p.src_pool + sb.off + (int64_t)g * (r + rv) * (lds + D);
  const uint16_t* sW = sh + (size_t)r * lds;
  const uint16_t* sUp = sW + (size_t)r * D;
  const uint16_t* sWp = sUp + (size_t)rv * lds;
  uint8_t* dh = p.dst_pool + db.off + (int64_t)g * kivi_head_bytes(nch, r, rv, D, BITS);
  uint16_t* KA = reinterpret_cast<uint16_t*>(dh + 16);
  uint16_t* KB = KA + (size_t)nch * 8 * ng8;
  uint8_t* KC = reinterpret_cast<uint8_t*>(KB + (size_t)nch * 8 * ng8);
  uint16_t* VA = reinterpret_cast<uint16_t*>(KC + (size_t)nch * 64 * BITS * ng8);
  uint16_t* VB = VA + (size_t)nch * ngv * 64;
  uint8_t* VC = reinterpret_cast<uint8_t*>(VB + (size_t)nch * ngv * 64);
  uint16_t* dW = reinterpret_cast<uint16_t*>(VC + (size_t)nch * 128 * BITS * ntv);
  uint16_t* dWp = dW + (size_t)r * D;

  float amax_k = 0.f, amax_v = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int t = 64 * c + lane;
    // ---- keys: rank component k over the chunk's tokens (padding ranks up to 8 ng8: 0)
    for (int k = wave; k < 8 * ng8; k += kKivThreads / 64) {
      const bool ok = k < r && t < T;
      const float x = ok ? bf16_at(sh, (size_t)k * lds + t) : 0.f;
      const float lo = wave_min(ok ? x : __builtin_huge_valf());
      const float hi = wave_max(ok ? x : -__builtin_huge_valf());
      _Float16 a16 = (_Float16)0.f, b16 = (_Float16)0.f;
      if (k < r && 64 * c < T) {
        a16 = (_Float16)__fdiv_rn(__fsub_rn(hi, lo), L);
        b16 = (_Float16)lo;
      }
      kc[k][lane] = ok ? (uint8_t)kiv_code(x, (float)b16, (float)a16, L) : 0;
      if (lane == 0) {
        KA[(size_t)c * 8 * ng8 + k] = f16_bits(a16);
        KB[(size_t)c * 8 * ng8 + k] = f16_bits(b16);
      }
      amax_k = fmaxf(amax_k, (float)a16);
    }
    // ---- values: token t over rank components 32 v .. 32 v + 31 (padding
    // components up to 16 ntv and padding tokens: codes 0, a = b = 0)
    if (wave < ngv) {
      const int v = wave, k0 = 32 * v, k1 = min(rv, k0 + 32), kp = min(16 * ntv, k0 + 32);
      _Float16 a16 = (_Float16)0.f, b16 = (_Float16)0.f;
      if (t < T) {
        float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
        for (int k = k0; k < k1; ++k) {
          const float x = bf16_at(sUp, (size_t)k * lds + t);
          lo = fminf(lo, x);
          hi = fmaxf(hi, x);
        }
        a16 = (_Float16)__fdiv_rn(__fsub_rn(hi, lo), L);
        b16 = (_Float16)lo;
        for (int k = k0; k < k1; ++k) vc[k][lane] = (uint8_t)kiv_code(bf16_at(sUp, (size_t)k * lds + t), (float)b16, (float)a16, L);
        for (int k = k1; k < kp; ++k) vc[k][lane] = 0;
      } else {
        for (int k = k0; k < kp; ++k) vc[k][lane] = 0;
      }
      VA[((size_t)c * ngv + v) * 64 + lane] = f16_bits(a16);
      VB[((size_t)c * ngv + v) * 64 + lane] = f16_bits(b16);
      amax_v = fmaxf(amax_v, (float)a16);
    }
    __syncthreads();
    // ---- key words: word (g8, col, m) holds ranks 8 g8 .. +7 of chunk token
    // 16 (col / 4) + 4 m + col % 4; 2-bit words (m = 2d, 2d + 1) share dword d
    {
      constexpr int DW = BITS == 4 ? 4 : 2;   // dwords per (g8, col)
      uint32_t* dst = reinterpret_cast<uint32_t*>(KC + (size_t)c * 64 * BITS * ng8);
      for (int x = tid; x < ng8 * 16 * DW; x += kKivThreads) {
        const int g8 = x / (16 * DW), col = (x / DW) % 16, d = x % DW;
        uint32_t w = 0;
#pragma unroll
        for (int u = 0; u < (BITS == 4 ? 1 : 2); ++u) {
          const int m = BITS == 4 ? d : 2 * d + u;
          const int tok = 16 * (col >> 2) + 4 * m + (col & 3);
#pragma unroll
          for (int i = 0; i < 8; ++i) w |= (uint32_t)kc[8 * g8 + i][tok] << code_shift<BITS>(u, i);
        }
        dst[x] = w;
      }
    }
    // ---- value words: tile kt, lane l holds rank 16 kt + l % 16 at chunk
    // tokens 16 (l / 16) + 8 s + i; 4-bit: dword s; 2-bit: words s = 0, 1 in one dword
    {
      constexpr int DW = BITS == 4 ? 2 : 1;   // dwords per (tile, lane)
      uint32_t* dst = reinterpret_cast<uint32_t*>(VC + (size_t)c * 128 * BITS * ntv);
      for (int x = tid; x < ntv * 64 * DW; x += kKivThreads) {
        const int kt = x / (64 * DW), l = (x / DW) % 64, d = x % DW;
        const int k = 16 * kt + (l & 15);
        uint32_t w = 0;
#pragma unroll
        for (int u = 0; u < (BITS == 4 ? 1 : 2); ++u) {
          const int s = BITS == 4 ? d : u;
#pragma unroll
          for (int i = 0; i < 8; ++i) w |= (uint32_t)vc[k][16 * (l >> 4) + 8 * s + i] << code_shift<BITS>(u, i);
        }
        dst[x] = w;
      }
    }
    __syncthreads();
  }
  // header: the largest key and value scale of the head
  amax_k = wave_max(amax_k);
  amax_v = wave_max(amax_v);
  if (lane == 0) {
    red[0][wave] = amax_k;
    red[1][wave] = amax_v;
  }
  __syncthreads();
  if (tid < 4) {
    float v = 0.f;
    if (tid < 2) {
#pragma unroll
      for (int w = 0; w < kKivThreads / 64; ++w) v = fmaxf(v, red[tid][w]);
    }
    reinterpret_cast<float*>(dh)[tid] = v;
  }
  for (int x = tid; x < r * D; x += kKivThreads) dW[x] = sW[x];
  for (int x = tid; x < rv * D; x += kKivThreads) dWp[x] = sWp[x];
}

}  // namespace

hipError_t launch_quantize_kivi(const QuantParams& p, int head_dim, int bits, hipStream_t s) {
  const int64_t wgs = (int64_t)p.n_blocks * p.n_kv_heads;
  if (wgs == 0) return hipSuccess;
  const dim3 grid((unsigned)wgs), block(kKivThreads);
  if (head_dim == 128 && bits == 4)
    hipLaunchKernelGGL((milo_kivi_quantize_kernel<128, 4>), grid, block, 0, s, p);
  else if (head_dim == 128 && bits == 2)
    hipLaunchKernelGGL((milo_kivi_quantize_kernel<128, 2>), grid, block, 0, s, p);
  else if (head_dim == 64 && bits == 4)
    hipLaunchKernelGGL((milo_kivi_quantize_kernel<64, 4>), grid, block, 0, s, p);
  else if (head_dim == 64 && bits == 2)
    hipLaunchKernelGGL((milo_kivi_quantize_kernel<64, 2>), grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace milo
