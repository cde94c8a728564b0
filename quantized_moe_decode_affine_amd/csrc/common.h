// Device helpers shared by the q4moe kernels (gfx950, wave64).
//
// Weight format: MLX affine 4-bit, group size 64 (lily README, introduction
// and "Requirements").  Column j of a row is the nibble at bits
// [4*(j%8), 4*(j%8)+4) of word j/8; w = scale*q + bias per 64-column group.
//
// Exact dequantization trick used by every product kernel: the bfloat16 bit
// pattern 0x4300 | q is exactly 128 + q for q in 0..15, so one AND-OR turns
// two nibbles of a word into two bfloat16 values.  With
//   P' = sum_j (128 + q_j) x_j  (bf16 x bf16 products, exact in fp32)
// a group contributes  scale*P' + (bias - 128*scale) * sum_j x_j, and
// bias - 128*scale is exact in fp32 (two bfloat16 values four binades apart).
// No weight is ever rounded.
//
// The nibble pairs of a word come out as (q0,q4), (q1,q5), (q2,q6), (q3,q7)
// (shift by 0, 4, 8, 12 then mask 0x000F000F), so activations are stored with
// the matching permutation of each 8-column block: (x0,x4),(x1,x5),(x2,x6),(x3,x7).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4moe {

constexpr int kGroup = 64;
constexpr int kWave = 64;
constexpr uint32_t kMagicPair = 0x43004300u;  // two bfloat16 128.0
constexpr uint32_t kNibblePairMask = 0x000F000Fu;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two nibbles of `word` (positions j and j+4, j = shift/4) as bfloat16 (128+q) pair.
__device__ __forceinline__ uint32_t nib_pair(uint32_t word, int shift) {
  return ((word >> shift) & kNibblePairMask) | kMagicPair;
}

// acc + a.lo*b.lo + a.hi*b.hi on packed bfloat16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// P' contribution of one code word against its 4 permuted activation pairs.
__device__ __forceinline__ float word_dot(uint32_t w, const uint32_t* xp, float acc) {
  acc = dot2_bf16(nib_pair(w, 0), xp[0], acc);
  acc = dot2_bf16(nib_pair(w, 4), xp[1], acc);
  acc = dot2_bf16(nib_pair(w, 8), xp[2], acc);
  acc = dot2_bf16(nib_pair(w, 12), xp[3], acc);
  return acc;
}

// Permute one 8-element bf16 block (4 dwords, natural order) into the pair order
// (x0,x4),(x1,x5),(x2,x6),(x3,x7).
__device__ __forceinline__ uint4 permute_block(uint4 v) {
  // byte selectors for v_perm_b32(hi_src, lo_src, sel): bytes 0-3 from lo_src, 4-7 from hi_src
  uint4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // x0 (v.x lo), x4 (v.z lo)
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // x1 (v.x hi), x5 (v.z hi)
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // x2, x6
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // x3, x7
  return r;
}

// Butterfly sum over groups of W consecutive lanes (W a power of two <= 64);
// every lane of a group ends with the group's total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Order-preserving map of a float to uint32 (larger float -> larger key); 0 is
// below every key of a non-NaN float.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace q4moe
