// chunk.hip -- gfx950 chunked-query attention over a block-wise low-rank KV
// cache (MFMA path).
//
// MILO (summary at paperlayer.ai/abs/2609.29913v1) keeps each block's keys and
// values as separate low-rank factors K_b ~= U_b W_b, V_b ~= U'_b W'_b ("4.2
// Block-wise Low-Rank Compression") and attends over the selected blocks
// ("4.4 MILO Workflow").  With Q new query tokens per sequence the G heads of
// a KV group give M = Q*G query rows, and each block is a chain of dense
// contractions, evaluated here in the transposed absorbed order
//     P^T = W Q^T            (r x M)     scaled by scale*log2(e)
//     S^T = U P^T            (T x M)     scores, log2 units
//     E^T = exp2(S^T - m)                online softmax per query row
//     Z^T = U'^T E^T         (r' x M)
//     O^T += W'^T Z^T        (d x M)
// on v_mfma_f32_32x32x16_bf16.  Each result tile is consumed as the next
// MFMA's operand straight from its accumulator registers: a 32x32 result
// holds, in lane l, column l%32 and rows {8a + 4(l/32) + b}, which is exactly
// an A/B operand whose K index runs over those rows.  The partner operand is
// read with the same K permutation: rank-major U^T and row-major W' come from
// LDS through ds_read_b64_tr_b16 (a 16-lane transpose read), U'^T rows are
// read directly.  Every query row's softmax state lives in the lanes that own
// its column, so rescaling is lane-local.
//
// Precision: P and Z are split into bf16 hi + lo parts (two MFMAs each), so
// scores and the value projection keep ~16 mantissa bits; e = exp2(s - m) is
// rounded to bf16 once (relative 2^-9 per weight, averaging out in the sum).
//
// Work unit = one workgroup of four waves: (sequence, KV head, 128 query rows,
// block range); wave w owns rows 32w..32w+31 of the tile.  The last range
// slot is the dense causal tail.  Units write (o~, m, l) partials that the
// merge kernel combines.
#include "device_common.h"
#include "kernels.h"

namespace milo {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kD = 128;            // head_dim of this kernel
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kTT = 64;            // tokens per staged U^T tile
constexpr int kUPitch = kTT + 8;   // LDS row pitch (elements) of the U^T tile
constexpr int kWPitch = kD + 8;    // LDS row pitch of W' and of the tail V tile
constexpr int kMaxR = 128;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator register v for a lane in half kg: (v/4)*8 + 4kg + v%4.
__device__ __forceinline__ int acc_row(int v, int kg) { return (v >> 2) * 8 + 4 * kg + (v & 3); }

// 8 consecutive accumulator registers (8c .. 8c+7) as a bf16 operand, split
// into hi = bf16(x) and lo = bf16(x - hi).  Operands are assembled from
// packed 32-bit words only: per-element __bf16 inserts into a vector were
// lowered by hipcc (ROCm 7.2) to a broadcast of element 0.
__device__ __forceinline__ void split_operand(const f32x16_t& acc, int c, bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = acc[8 * c + 2 * k], x1 = acc[8 * c + 2 * k + 1];
    h[k] = pack_bf16(x0, x1);
    l[k] = pack_bf16(x0 - bf_lo(h[k]), x1 - bf_hi(h[k]));
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}
__device__ __forceinline__ bf16x8_t to_operand(const f32x16_t& acc, int c) {
  u32x4_t h;
#pragma unroll
  for (int k = 0; k < 4; ++k) h[k] = pack_bf16(acc[8 * c + 2 * k], acc[8 * c + 2 * k + 1]);
  return __builtin_bit_cast(bf16x8_t, h);
}

// Operand whose K index follows the accumulator row permutation, read from a
// K-major LDS array X (row = K index, pitch in elements, columns contiguous):
// slot s of lane l <- X[row0 + 4(l/32) + 8(s/4) + s%4][col0 + l%32].  Two
// transposing 8-byte reads per lane.
__device__ __forceinline__ bf16x8_t tr_operand(const uint16_t* X, int pitch, int row0, int col0,
                                               int lane) {
  const int kg = lane >> 5;
  const int r = row0 + 4 * kg + ((lane & 15) >> 2);
  const int c = col0 + 4 * (lane & 3) + 16 * ((lane >> 4) & 1);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(X + r * pitch + c));
  const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(X + (r + 8) * pitch + c));
  const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
  const u32x4_t w = {w0[0], w0[1], w1[0], w1[1]};
  return __builtin_bit_cast(bf16x8_t, w);
}

struct LdsLayout {
  uint16_t wp[kMaxR * kWPitch];    // W' (rank' rows, zero-padded to a multiple of 32)
  uint16_t u[kMaxR * kUPitch];     // U^T token tile, or the tail V tile
};

// Stage rows [0, nrows_pad) x `chunks` 16-byte chunks of a row-major source
// (row stride src_ld elements, starting at byte offset base) into LDS with
// pitch `pitch`; rows >= nrows are written as zeros.
__device__ __forceinline__ void stage_rows(rsrc_t rs, uint32_t base, int src_ld, int nrows,
                                           int nrows_pad, int chunks, int col0, uint16_t* dst,
                                           int pitch, int tid) {
  for (int id = tid; id < nrows_pad * chunks; id += kWaves * 64) {
    const int row = id / chunks, ch = id - row * chunks;
    u32x4_t v = {0, 0, 0, 0};
    if (row < nrows) v = bld16(rs, (uint32_t)(row * src_ld + col0 + ch * 8) * 2, base);
    *reinterpret_cast<u32x4_t*>(dst + row * pitch + ch * 8) = v;
  }
}

template <int G>
__global__ __launch_bounds__(256) void milo_chunk_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) LdsLayout lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, kg = lane >> 5;
  const int S = p.n_ranges + 1;
  const int unit = blockIdx.x;
  const int slot = unit % S;
  int rest = unit / S;
  const int qt = rest % p.n_qtiles;
  rest /= p.n_qtiles;
  const int g = rest % p.n_kv_heads, i = rest / p.n_kv_heads;
  const int MQ = p.q_len * G;
  const int m0 = qt * (kWaves * kRowsPerWave) + wave * kRowsPerWave;
  const int m_l = m0 + (lane & 31);   // this lane's query row (column of every tile)
  const bool row_ok = m_l < MQ;
  const int j_l = m_l / G, hl = m_l - j_l * G;

  const int b0 = p.seq_blocks[i];
  const int nb = min(max(p.seq_blocks[i + 1] - b0, 0), p.max_blocks);
  const int blk_lo = slot * p.blocks_per_range;
  const int blk_hi = min(nb, blk_lo + p.blocks_per_range);
  const bool tail = slot == p.n_ranges;
  if (!tail && blk_lo >= blk_hi) return;   // empty range: the merge skips it

  // Q^T operand: qv[kk] = q[row m_l][16kk + 8kg .. +8]
  u32x4_t qv[kD / 16];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           (((int64_t)i * p.q_len + j_l) * p.n_q_heads + g * G + hl) * kD;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      qv[kk] = u32x4_t{0, 0, 0, 0};
      if (row_ok) qv[kk] = ld16(qrow + 16 * kk + 8 * kg);
    }
  }

  f32x16_t O[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[dt][v] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  // Online softmax of one 32-token x 32-row score tile (log2 units, masked
  // entries -inf); rescales O (and Z when given) and returns e as operands.
  auto softmax_tile = [&](f32x16_t& s, f32x16_t* Z, int nz, bf16x8_t (&eb)[2]) {
    float mx = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
    {
      float a = mx, b = mx;
      swap32(a, b);
      mx = fmaxf(a, b);
    }
    const float mn = fmaxf(m_run, mx);
    const float alpha = (mn == kNegInf) ? 1.f : fast_exp2(m_run - mn);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[dt][v] *= alpha;
#pragma unroll
      for (int zt = 0; zt < kMaxR / 32; ++zt)
        if (zt < nz)
#pragma unroll
          for (int v = 0; v < 16; ++v) Z[zt][v] *= alpha;
    }
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float e = (mn == kNegInf) ? 0.f : fast_exp2(s[v] - mn);
      s[v] = e;
      sum += e;
    }
    l_run = l_run * alpha + sum;
    m_run = mn;
    eb[0] = to_operand(s, 0);
    eb[1] = to_operand(s, 1);
  };

  if (!tail) {
    f32x16_t Z[kMaxR / 32];
    for (int b = blk_lo; b < blk_hi; ++b) {
      const milo_block blk = p.blocks[b0 + b];
      const int T = max(blk.n_tok, 0), ld = blk.ld_tok;
      const int r = min(max(blk.rank_k, 0), kD), rv = min(max(blk.rank_v, 0), kD);
      const int nrt = (r + 31) / 32, nvt = (rv + 31) / 32;
      const uint16_t* head = reinterpret_cast<const uint16_t*>(p.pool) + blk.off +
                             (int64_t)g * (r + rv) * (ld + kD);
      const rsrc_t rs = make_rsrc(head, (uint32_t)((r + rv) * (ld + kD)) * 2);
      const uint32_t w_off = (uint32_t)(r * ld) * 2;
      const uint32_t v_off = w_off + (uint32_t)(r * kD) * 2;
      const uint32_t wp_off = v_off + (uint32_t)(rv * ld) * 2;

      __syncthreads();   // previous block's LDS reads are done
      stage_rows(rs, wp_off, kD, rv, nvt * 32, kD / 8, 0, lds.wp, kWPitch, tid);

      // ---- P^T = W Q^T per 32-rank tile, scaled, split into hi/lo operands
      bf16x8_t ph[kMaxR / 32][2], pl[kMaxR / 32][2];
#pragma unroll
      for (int rt = 0; rt < kMaxR / 32; ++rt) {
        if (rt < nrt) {
          f32x16_t acc;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] = 0.f;
          const int wrow = 32 * rt + (lane & 31);
#pragma unroll
          for (int kk = 0; kk < kD / 16; ++kk) {
            u32x4_t wa = {0, 0, 0, 0};
            if (wrow < r) wa = bld16(rs, (uint32_t)(wrow * kD + 16 * kk + 8 * kg) * 2, w_off);
            acc = mfma(__builtin_bit_cast(bf16x8_t, wa), __builtin_bit_cast(bf16x8_t, qv[kk]), acc);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acc[v] = (32 * rt + acc_row(v, kg) < r) ? acc[v] * p.scale_log2 : 0.f;
          split_operand(acc, 0, ph[rt][0], pl[rt][0]);
          split_operand(acc, 1, ph[rt][1], pl[rt][1]);
        }
      }
#pragma unroll
      for (int zt = 0; zt < kMaxR / 32; ++zt)
#pragma unroll
        for (int v = 0; v < 16; ++v) Z[zt][v] = 0.f;

      for (int t0 = 0; t0 < T; t0 += kTT) {
        __syncthreads();   // previous tile's reads of lds.u are done
        stage_rows(rs, (uint32_t)t0 * 2, ld, r, nrt * 32, kTT / 8, 0, lds.u, kUPitch, tid);
        __syncthreads();
#pragma unroll
        for (int st = 0; st < kTT / 32; ++st) {
          const int tb = t0 + 32 * st;
          if (tb >= T) break;
          // U'^T operands for this sub-tile: rank' row 32vt + l%32, tokens
          // tb + 16c + 4kg + {0..3} and + 8 (masked past the block end)
          bf16x8_t ua[kMaxR / 32][2];
#pragma unroll
          for (int vt = 0; vt < kMaxR / 32; ++vt) {
            if (vt < nvt) {
              const int vrow = 32 * vt + (lane & 31);
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const int tk = tb + 16 * c + 4 * kg;
                u32x2_t lo2 = {0, 0}, hi2 = {0, 0};
                if (vrow < rv) {
                  const int off = (int)(v_off + (uint32_t)(vrow * ld + tk) * 2);
                  lo2 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
                  hi2 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 16, 0, 0));
                }
                if (tb + 32 > T) {   // zero tokens past the block end (padding may be NaN)
#pragma unroll
                  for (int h2 = 0; h2 < 2; ++h2) {
                    const int ta = tk + 2 * h2, tb2 = tk + 8 + 2 * h2;
                    lo2[h2] &= (ta < T ? 0xffffu : 0u) | (ta + 1 < T ? 0xffff0000u : 0u);
                    hi2[h2] &= (tb2 < T ? 0xffffu : 0u) | (tb2 + 1 < T ? 0xffff0000u : 0u);
                  }
                }
                const u32x4_t w4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
                ua[vt][c] = __builtin_bit_cast(bf16x8_t, w4);
              }
            }
          }
          // ---- S^T = U P^T (hi + lo)
          f32x16_t s;
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
          for (int rt = 0; rt < kMaxR / 32; ++rt) {
            if (rt < nrt) {
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const bf16x8_t a = tr_operand(lds.u, kUPitch, 32 * rt + 16 * c, 32 * st, lane);
                s = mfma(a, ph[rt][c], s);
                s = mfma(a, pl[rt][c], s);
              }
            }
          }
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (tb + acc_row(v, kg) >= T) s[v] = kNegInf;
          bf16x8_t eb[2];
          softmax_tile(s, Z, nvt, eb);
          // ---- Z^T += U'^T E^T
#pragma unroll
          for (int vt = 0; vt < kMaxR / 32; ++vt) {
            if (vt < nvt) {
              Z[vt] = mfma(ua[vt][0], eb[0], Z[vt]);
              Z[vt] = mfma(ua[vt][1], eb[1], Z[vt]);
            }
          }
        }
      }
      // ---- O^T += W'^T Z^T (hi + lo)
      __syncthreads();   // W' staged (and visible) before the transposing reads
#pragma unroll
      for (int vt = 0; vt < kMaxR / 32; ++vt) {
        if (vt < nvt) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            bf16x8_t zh, zl;
            split_operand(Z[vt], c, zh, zl);
#pragma unroll
            for (int dt = 0; dt < kD / 32; ++dt) {
              const bf16x8_t a = tr_operand(lds.wp, kWPitch, 32 * vt + 16 * c, 32 * dt, lane);
              O[dt] = mfma(a, zh, O[dt]);
              O[dt] = mfma(a, zl, O[dt]);
            }
          }
        }
      }
    }
  } else {
    // ---- dense causal tail: token l is visible to query j iff l <= L - Q + j
    const int cap = p.tail_cap;
    const int L = min(max(p.tail_len[i], 0), cap);
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(p.k_tail) + ((size_t)i * p.n_kv_heads + g) * cap * kD;
    const uint16_t* vtp = reinterpret_cast<const uint16_t*>(p.v_tail) + ((size_t)i * p.n_kv_heads + g) * cap * kD;
    const rsrc_t rk = make_rsrc(kt, (uint32_t)(cap * kD) * 2);
    const rsrc_t rvv = make_rsrc(vtp, (uint32_t)(cap * kD) * 2);
    const int vis = L - p.q_len + j_l;   // last visible tail token of this row
    for (int t0 = 0; t0 < L; t0 += 32) {
      __syncthreads();
      stage_rows(rvv, (uint32_t)(t0 * kD) * 2, kD, min(32, L - t0), 32, kD / 8, 0, lds.u, kWPitch, tid);
      __syncthreads();
      // S^T = K_tail q^T, K = d
      f32x16_t s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.f;
      const int krow = t0 + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) {
        u32x4_t ka = {0, 0, 0, 0};
        if (krow < L) ka = bld16(rk, (uint32_t)(krow * kD + 16 * kk + 8 * kg) * 2, 0);
        s = mfma(__builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qv[kk]), s);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + acc_row(v, kg);
        s[v] = (t < L && t <= vis) ? s[v] * p.scale_log2 : kNegInf;
      }
      bf16x8_t eb[2];
      softmax_tile(s, nullptr, 0, eb);
      // O^T += V_tail^T E^T
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const bf16x8_t a = tr_operand(lds.u, kWPitch, 16 * c, 32 * dt, lane);
          O[dt] = mfma(a, eb[c], O[dt]);
        }
    }
  }

  // ---- partials: row m_l of this unit's record, o~ (d = 32dt + acc_row) and (m, l)
  {
    float a = l_run, b = l_run;
    swap32(a, b);
    l_run = a + b;
  }
  if (row_ok) {
    const size_t rec = ((size_t)((i * p.n_kv_heads + g) * S + slot)) * MQ + m_l;
    float* po = p.part.o + rec * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4_t*>(po + 32 * dt + q4 * 8 + 4 * kg) =
            f32x4_t{O[dt][4 * q4], O[dt][4 * q4 + 1], O[dt][4 * q4 + 2], O[dt][4 * q4 + 3]};
    if (kg == 0) {
      p.part.ml[rec * 2 + 0] = m_run;
      p.part.ml[rec * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_chunk(const ChunkParams& p, int group, hipStream_t s) {
  const int64_t units = (int64_t)p.batch * p.n_kv_heads * p.n_qtiles * (p.n_ranges + 1);
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)units), block(64 * kWaves);
  switch (group) {
#define MILO_G(GG) \
  case GG: hipLaunchKernelGGL((milo_chunk_kernel<GG>), grid, block, 0, s, p); break;
    MILO_G(1) MILO_G(2) MILO_G(3) MILO_G(4) MILO_G(5) MILO_G(6) MILO_G(7) MILO_G(8)
#undef MILO_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace milo
