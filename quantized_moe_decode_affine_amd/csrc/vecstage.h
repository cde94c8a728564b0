// Staging of activation vectors into LDS for the Q4 GEMV-style kernels, and
// the per-lane chunk dot product that consumes them.
//
// A "chunk" is 32 consecutive columns: one uint4 of codes (4 words) and half
// of a 64-column quantization group.  An activation vector is staged chunk by
// chunk as permuted bfloat16 pairs (see common.h): NV = 1 for a bf16 input,
// NV = 2 for an fp32 input split exactly into hi + lo bfloat16 parts (the
// residual is below 2^-17 of each element).  Alongside each chunk we keep the
// fp32 sum of the staged values, used by the bias/offset term.
#pragma once

#include "common.h"

namespace q4moe {

// dwords per staged chunk: NV*16 pair words plus 4 words of padding so that
// lanes reading consecutive chunks hit different LDS banks.
template <int NV>
__host__ __device__ constexpr int chunk_stride() { return NV * 16 + 4; }

// Stage chunk c of a bf16 vector: its 32 values as permuted pairs at dst, their sum at *sum.
__device__ __forceinline__ void stage_bf16_chunk(const uint16_t* __restrict__ x, int c, uint32_t* dst, float* sum) {
  const uint4* src = reinterpret_cast<const uint4*>(x) + 4 * c;
  float s = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint4 v = src[b];
    s += (bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16)) +
         (bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16)) +
         (bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16)) +
         (bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16));
    *reinterpret_cast<uint4*>(dst + 4 * b) = permute_block(v);
  }
  *sum = s;
}

// Stage a bf16 vector of C chunks (C*32 values) into vp (pairs) and vs (sums).
__device__ __forceinline__ void stage_bf16_vector(const uint16_t* __restrict__ x, int C,
                                                  uint32_t* vp, float* vs) {
  for (int c = threadIdx.x; c < C; c += blockDim.x) stage_bf16_chunk(x, c, vp + c * chunk_stride<1>(), vs + c);
}

// Stage chunk c of an fp32 vector as hi/lo bfloat16 parts at dst, the sum of the parts at *sum.
__device__ __forceinline__ void stage_f32_split_chunk(const float* __restrict__ a, int c, uint32_t* dst, float* sum) {
  const float4* src = reinterpret_cast<const float4*>(a) + 8 * c;
  float s = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float4 u = src[2 * b], w = src[2 * b + 1];
    float v[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hi[j] = f32_to_bf16_bits(v[j]);
      float h = bf16_bits_to_f32(hi[j]);
      lo[j] = f32_to_bf16_bits(v[j] - h);
      s += h + bf16_bits_to_f32(lo[j]);
    }
    uint4 ph, pl;
    ph.x = hi[0] | (hi[4] << 16); ph.y = hi[1] | (hi[5] << 16);
    ph.z = hi[2] | (hi[6] << 16); ph.w = hi[3] | (hi[7] << 16);
    pl.x = lo[0] | (lo[4] << 16); pl.y = lo[1] | (lo[5] << 16);
    pl.z = lo[2] | (lo[6] << 16); pl.w = lo[3] | (lo[7] << 16);
    *reinterpret_cast<uint4*>(dst + 4 * b) = ph;
    *reinterpret_cast<uint4*>(dst + 16 + 4 * b) = pl;
  }
  *sum = s;
}

// Stage an fp32 vector of C chunks as hi/lo bfloat16 parts.
__device__ __forceinline__ void stage_f32_split_vector(const float* __restrict__ a, int C,
                                                       uint32_t* vp, float* vs) {
  for (int c = threadIdx.x; c < C; c += blockDim.x) stage_f32_split_chunk(a, c, vp + c * chunk_stride<2>(), vs + c);
}

// P' of one chunk: sum over its 32 columns of (128 + q) * v.
template <int NV>
__device__ __forceinline__ float chunk_pdot(uint4 codes, const uint32_t* vchunk) {
  uint32_t v[16];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint4 t = *reinterpret_cast<const uint4*>(vchunk + 4 * b);
    v[4 * b] = t.x; v[4 * b + 1] = t.y; v[4 * b + 2] = t.z; v[4 * b + 3] = t.w;
  }
  float p0 = word_dot(codes.x, v + 0, 0.f);
  float p1 = word_dot(codes.y, v + 4, 0.f);
  p0 = word_dot(codes.z, v + 8, p0);
  p1 = word_dot(codes.w, v + 12, p1);
  if constexpr (NV == 2) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint4 t = *reinterpret_cast<const uint4*>(vchunk + 16 + 4 * b);
      v[4 * b] = t.x; v[4 * b + 1] = t.y; v[4 * b + 2] = t.z; v[4 * b + 3] = t.w;
    }
    p0 = word_dot(codes.x, v + 0, p0);
    p1 = word_dot(codes.y, v + 4, p1);
    p0 = word_dot(codes.z, v + 8, p0);
    p1 = word_dot(codes.w, v + 12, p1);
  }
  return p0 + p1;
}

// Contribution of a group-aligned chunk pair or single chunk: scale*P' + (bias-128*scale)*sum.
__device__ __forceinline__ float affine_term(float p, float vsum, uint32_t s_bits, uint32_t b_bits) {
  float s = bf16_bits_to_f32(s_bits);
  float c = bf16_bits_to_f32(b_bits) - 128.0f * s;  // exact
  return fmaf(s, p, c * vsum);
}

}  // namespace q4moe
