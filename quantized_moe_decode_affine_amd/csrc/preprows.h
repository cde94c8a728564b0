// fp16 copies of matrix rows for the grouped GEMM's A operand (the token rows of a
// prefill chunk, the SwiGLU outputs), shared by the launch of their own in gemm.hip and
// the one that runs them beside the sort's rank step in route.hip.
#pragma once

#include <stdint.h>

#include <type_traits>

#include "common.h"

namespace q4moe {
namespace prep {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Load 8 consecutive elements of a row as fp32 (bf16 bits or fp32 input).
__device__ __forceinline__ void load8(const uint16_t* src, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
    v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
  }
}
// fp16 values stored with a power of two per four columns (value = fp16 * 2^e).
struct f16x_t {
  uint16_t bits;
};
__device__ __forceinline__ void load8(const f16x_t* src, const int8_t* ex, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  const uint32_t e2 = *reinterpret_cast<const uint16_t*>(ex);  // the exponents of columns 0-3 and 4-7
  const int e0 = (int8_t)(e2 & 0xFFu), e1 = (int8_t)(e2 >> 8);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half2_t h = __builtin_bit_cast(half2_t, w[j]);
    const int e = j < 2 ? e0 : e1;
    v[2 * j] = ldexpf((float)h[0], e);
    v[2 * j + 1] = ldexpf((float)h[1], e);
  }
}
__device__ __forceinline__ void load8(const float* src, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Rows whose values come from K-split partial sums: row r >= from is silu(g) * u with
// g = sum_k part[k*stride + (r-from)*2K + j] and u the same at + K (k in order).
struct SplitRows {
  const float* part;
  int64_t from;    // no such rows: INT64_MAX
  int64_t stride;  // floats between ranges
  int ks;
};

// fp16 copy of rows for the MFMA A operand, one wave per row.  The row's largest
// magnitude M picks e with M * 2^-e in [256, 512) (e = 0 for an all-zero row); the
// row is written as fp16(x * 2^-e) with each 8-element block in the pair order
// (x0,x4),(x1,x5),(x2,x6),(x3,x7), e goes to exps[row], and the sums of each 64-wide
// group of the fp16 values are split into two fp16 parts: sums[row][part][g], with
// the groups padded with zeros to Gp.  With In = f16x_t, in_exp holds the input's powers
// of two, [rows][K/4].
template <typename In>
__device__ __forceinline__ void prep_rows_body(const In* __restrict__ A, int64_t rows, int K, int Gp,
                                               uint16_t* __restrict__ out, uint16_t* __restrict__ sums,
                                               int32_t* __restrict__ exps, SplitRows sp, int64_t block, int64_t nblocks,
                                               const int8_t* __restrict__ in_exp = nullptr) {
  const int lane = lane_id();
  const int nblk = K >> 3, G = K >> 6;
  const int64_t wstride = nblocks * (blockDim.x / kWave);
  for (int64_t r = block * (blockDim.x / kWave) + threadIdx.x / kWave; r < rows; r += wstride) {
    const In* row = A + r * K;
    // rows from sp.from on: the SwiGLU of K-split gate and up sums, added in range order
    const float* prow = r >= sp.from ? sp.part + (r - sp.from) * 2 * K : nullptr;
    auto load = [&](int b, float (&v)[8]) __attribute__((always_inline)) {
      if (prow) {
        float g[8], u[8], t[8];
        load8(prow + b * 8, g);
        load8(prow + K + b * 8, u);
        for (int k = 1; k < sp.ks; ++k) {
          load8(prow + k * sp.stride + b * 8, t);
#pragma unroll
          for (int j = 0; j < 8; ++j) g[j] += t[j];
          load8(prow + k * sp.stride + K + b * 8, t);
#pragma unroll
          for (int j = 0; j < 8; ++j) u[j] += t[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = silu(g[j]) * u[j];
      } else if constexpr (std::is_same_v<In, f16x_t>) {
        load8(row + b * 8, in_exp + (r * K + b * 8) / 4, v);
      } else {
        load8(row + b * 8, v);
      }
    };
    // A row of at most 64 blocks is read once and kept in registers; a longer one is
    // read again for the conversion.
    const bool one = nblk <= kWave;
    float vk[8] = {};
    uint32_t mx = 0;  // largest |x| as float bits (non-negative floats order as integers)
    if (one) {
      if (lane < nblk) load(lane, vk);
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = max(mx, __float_as_uint(fabsf(vk[j])));
    } else {
      for (int b = lane; b < nblk; b += kWave) {
        float v[8];
        load(b, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = max(mx, __float_as_uint(fabsf(v[j])));
      }
    }
    mx = wave_max_u32(mx);
    const float m = __uint_as_float(mx);
    int e = 0;
    if (m > 0.0f && m <= 3.0e38f) {
      int ex;
      frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
      e = ex - 9;
    }
    uint16_t* orow = out + r * K;
    uint16_t* srow = sums + r * 2 * Gp;
    for (int b0 = 0; b0 < nblk; b0 += kWave) {
      const int b = b0 + lane;
      float gs = 0.0f;
      if (b < nblk) {
        float v[8];
        if (one) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = vk[j];
        } else {
          load(b, v);
        }
        _Float16 h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          h[j] = (_Float16)ldexpf(v[j], -e);
          gs += (float)h[j];
        }
        uint4 o;
        o.x = __builtin_bit_cast(uint32_t, half2_t{h[0], h[4]});
        o.y = __builtin_bit_cast(uint32_t, half2_t{h[1], h[5]});
        o.z = __builtin_bit_cast(uint32_t, half2_t{h[2], h[6]});
        o.w = __builtin_bit_cast(uint32_t, half2_t{h[3], h[7]});
        *reinterpret_cast<uint4*>(orow + b * 8) = o;
      }
      gs = group_sum<8>(gs);  // the 8 blocks of a group sit in 8 consecutive lanes
      if (b < nblk && (b & 7) == 0) {
        const _Float16 hi = (_Float16)gs;
        const _Float16 lo = (_Float16)(gs - (float)hi);
        srow[b >> 3] = __builtin_bit_cast(uint16_t, hi);
        srow[Gp + (b >> 3)] = __builtin_bit_cast(uint16_t, lo);
      }
    }
    if (lane < Gp - G) {
      srow[G + lane] = 0;
      srow[Gp + G + lane] = 0;
    }
    if (lane == 0) exps[r] = e;
  }
}

}  // namespace prep
}  // namespace q4moe
