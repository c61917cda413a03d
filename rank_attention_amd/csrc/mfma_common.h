// mfma_common.h -- gfx950 matrix-core operand helpers and the LDS DMA
// shared by the MFMA attention kernels (chunked query, decode).
#pragma once

#include "device_common.h"

namespace milo {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

__device__ __forceinline__ f32x4_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                   __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// Two stacked 16x16 results (rows 0-15 in x, 16-31 in y) as a K = 32 bf16
// operand, split into hi = bf16(v) and lo = bf16(v - hi).  Operands are
// assembled from packed 32-bit words only: per-element __bf16 inserts into
// a vector were lowered by hipcc (ROCm 7.2) to a broadcast of element 0.
__device__ __forceinline__ void split_pair(const f32x4_t& x, const f32x4_t& y, u32x4_t& hi, u32x4_t& lo) {
  hi[0] = pack_bf16(x[0], x[1]);
  hi[1] = pack_bf16(x[2], x[3]);
  hi[2] = pack_bf16(y[0], y[1]);
  hi[3] = pack_bf16(y[2], y[3]);
  lo[0] = pack_bf16(x[0] - bf_lo(hi[0]), x[1] - bf_hi(hi[0]));
  lo[1] = pack_bf16(x[2] - bf_lo(hi[1]), x[3] - bf_hi(hi[1]));
  lo[2] = pack_bf16(y[0] - bf_lo(hi[2]), y[1] - bf_hi(hi[2]));
  lo[3] = pack_bf16(y[2] - bf_lo(hi[3]), y[3] - bf_hi(hi[3]));
}
// One 16x16 result as a K = 16 operand, split hi + lo.
__device__ __forceinline__ void split_one(const f32x4_t& x, u32x2_t& hi, u32x2_t& lo) {
  hi[0] = pack_bf16(x[0], x[1]);
  hi[1] = pack_bf16(x[2], x[3]);
  lo[0] = pack_bf16(x[0] - bf_lo(hi[0]), x[1] - bf_hi(hi[0]));
  lo[1] = pack_bf16(x[2] - bf_lo(hi[1]), x[3] - bf_hi(hi[1]));
}
__device__ __forceinline__ u32x4_t pack_pair(const f32x4_t& x, const f32x4_t& y) {
  return u32x4_t{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(y[0], y[1]),
                 pack_bf16(y[2], y[3])};
}

__device__ __forceinline__ u32x2_t tr_read(const char* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

// Buffer resource words (base, no stride, `bytes` records, raw dword
// format) of a wave-uniform range, for the LDS DMA below.
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu,
                 (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}
// 16 bytes per lane from the buffer into LDS at lds + 16*lane (lds
// wave-uniform, passed in M0).  Lanes with !ok read past the resource's
// size and write zeros.  Issued from asm so that the compiler does not
// track it: it cannot tell which LDS buffer the load writes and would wait
// for every load in flight before each LDS read.  The waits are explicit
// (wait_barrier) instead.  The compiler does not insert hazard wait states
// for an asm statement's operands, so the asm holds them: a VMEM
// instruction reading an SGPR that a VALU instruction wrote (the resource
// words come from v_readfirstlane) needs 5 wait states, one reading M0
// after an SALU write needs 1; s_nop 4 gives 5.
__device__ __forceinline__ void dma16(const u32x4_t& rs, char* lds, uint32_t off, bool ok) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds));
  const uint32_t voff = ok ? off : 0x80000000u;
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "{m0}"(m0)
               : "memory");
}
// x, hidden from the optimizer: per-lane LDS and DMA offsets derived from it
// are recomputed where they are used instead of being hoisted out of the
// loops and kept live (they would take ~40 registers for the whole unit).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

}  // namespace milo
