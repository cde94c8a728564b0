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

// 8-bit codes against a staged chunk.  A code q in 0..255 is an integer of at most 8
// significant bits, so it is exact in bfloat16 (the high half of its fp32 value); the
// pairs (q_j, q_{j+4}) of an 8-code block (words w0 = codes 0..3, w1 = codes 4..7, byte
// j of a word = code j) match the staged activation pairs (x_j, x_{j+4}).
__device__ __forceinline__ void q8_block_pairs(uint32_t w0, uint32_t w1, uint32_t (&pr)[4]) {
  // (one v_cvt_f32_ubyteN each)
  const float a0 = (float)(w0 & 0xFFu), b0 = (float)(w1 & 0xFFu);
  const float a1 = (float)((w0 >> 8) & 0xFFu), b1 = (float)((w1 >> 8) & 0xFFu);
  const float a2 = (float)((w0 >> 16) & 0xFFu), b2 = (float)((w1 >> 16) & 0xFFu);
  const float a3 = (float)(w0 >> 24), b3 = (float)(w1 >> 24);
  // high halves of two fp32 values as one bf16 pair (lo from the first)
  pr[0] = __builtin_amdgcn_perm(__float_as_uint(b0), __float_as_uint(a0), 0x07060302u);
  pr[1] = __builtin_amdgcn_perm(__float_as_uint(b1), __float_as_uint(a1), 0x07060302u);
  pr[2] = __builtin_amdgcn_perm(__float_as_uint(b2), __float_as_uint(a2), 0x07060302u);
  pr[3] = __builtin_amdgcn_perm(__float_as_uint(b3), __float_as_uint(a3), 0x07060302u);
}

// sum over a chunk's 32 columns of q * v for 8-bit codes c (32 bytes: c0 = codes 0..15,
// c1 = codes 16..31) against a chunk staged with NV parts.
template <int NV>
__device__ __forceinline__ float q8_chunk_pdot(uint4 c0, uint4 c1, const uint32_t* vchunk) {
  const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {  // 8-code blocks
    uint32_t pr[4];
    q8_block_pairs(w[2 * b], w[2 * b + 1], pr);
#pragma unroll
    for (int part = 0; part < NV; ++part) {
      const uint4 t = *reinterpret_cast<const uint4*>(vchunk + 16 * part + 4 * b);
      p0 = dot2_bf16(pr[0], t.x, p0);
      p1 = dot2_bf16(pr[1], t.y, p1);
      p0 = dot2_bf16(pr[2], t.z, p0);
      p1 = dot2_bf16(pr[3], t.w, p1);
    }
  }
  return p0 + p1;
}

// The same against one bf16 chunk already in registers (16 pair words).
__device__ __forceinline__ float q8_chunk_pdot_regs(uint4 c0, uint4 c1, const uint32_t (&v)[16]) {
  const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t pr[4];
    q8_block_pairs(w[2 * b], w[2 * b + 1], pr);
    p0 = dot2_bf16(pr[0], v[4 * b], p0);
    p1 = dot2_bf16(pr[1], v[4 * b + 1], p1);
    p0 = dot2_bf16(pr[2], v[4 * b + 2], p0);
    p1 = dot2_bf16(pr[3], v[4 * b + 3], p1);
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
