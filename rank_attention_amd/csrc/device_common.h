// device_common.h -- wave64 helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace milo {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte global load that the compiler may not split or reorder past stores.
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ f32x4_t ld16f(const void* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}
// 16-byte load of data read once per launch, wave-coalesced (a wave's lanes
// cover whole cache lines): marked non-temporal, so the stream does not
// displace cached data.  Not for lane-strided reads, whose lines are
// reused by the lane's next loads.
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Raw buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros instead of faulting.  The third dword selects the 32-bit data
// format required for untyped loads on this ISA.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte load at byte offset voff (per lane) + soff (wave-uniform).
__device__ __forceinline__ u32x4_t bld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// d = a.lo*b.lo + a.hi*b.hi + c, bf16 pairs, fp32 accumulate (exact products).
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// d = a.lo*b.lo + a.hi*b.hi + c, fp16 pairs, fp32 accumulate (exact products).
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// Two fp32 values to a packed fp16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 values to a packed bf16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Interleave the bf16 halves of two dwords: lo = (x.lo, y.lo), hi = (x.hi, y.hi).
__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
// DPP controls (GFX9 encoding)
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;    // lane i <-> 7-i inside each group of 8
constexpr int kRowRor8 = 0x128;       // lane i <-> i^8 inside each row of 16

// Swap halves across rows: returns {x', y'} with
//   permlane16: x' = rows (x0, y0, x2, y2), y' = rows (x1, y1, x3, y3)
//   permlane32: x' = halves (x_lo, y_lo),   y' = halves (x_hi, y_hi)
__device__ __forceinline__ void swap16(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Lane 0's value, as a wave-uniform (scalar register) value.
__device__ __forceinline__ float uniform_f32(float v) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kHalfMirror>(v));
  v = fmaxf(v, dpp<kRowRor8>(v));
  float a = v, b = v;
  swap16(a, b);
  v = fmaxf(a, b);
  a = v; b = v;
  swap32(a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp<kQuadXor1>(v));
  v = fminf(v, dpp<kQuadXor2>(v));
  v = fminf(v, dpp<kHalfMirror>(v));
  v = fminf(v, dpp<kRowRor8>(v));
  float a = v, b = v;
  swap16(a, b);
  v = fminf(a, b);
  a = v; b = v;
  swap32(a, b);
  return fminf(a, b);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kHalfMirror>(v);
  v += dpp<kRowRor8>(v);
  float a = v, b = v;
  swap16(a, b);
  v = a + b;
  a = v; b = v;
  swap32(a, b);
  return a + b;
}

// One butterfly stage inside a row: the lane whose BIT is set keeps b, its
// partner keeps a; each receives the partner's copy of what it keeps.
template <int CTRL, int BIT>
__device__ __forceinline__ float keep_add(float a, float b, int lane) {
  const bool upper = (lane & BIT) != 0;
  const float send = upper ? a : b;
  const float keep = upper ? b : a;
  return keep + dpp<CTRL>(send);
}

// Transposing reduction of 64 per-lane partial sums across the 64 lanes of a
// wave: on return, lane l holds sum over all lanes of v[l].  v is destroyed.
__device__ __forceinline__ float reduce_transpose64(float (&v)[64], int lane) {
#pragma unroll
  for (int j = 0; j < 32; ++j) { swap32(v[j], v[j + 32]); v[j] += v[j + 32]; }
#pragma unroll
  for (int j = 0; j < 16; ++j) { swap16(v[j], v[j + 16]); v[j] += v[j + 16]; }
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = keep_add<kRowRor8, 8>(v[j], v[j + 8], lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = keep_add<kHalfMirror, 4>(v[j], v[j + 4], lane);
#pragma unroll
  for (int j = 0; j < 2; ++j) v[j] = keep_add<kQuadXor2, 2>(v[j], v[j + 2], lane);
  return keep_add<kQuadXor1, 1>(v[0], v[1], lane);
}

}  // namespace milo
