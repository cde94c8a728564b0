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

// kMagicPair in a VGPR, from an asm the compiler cannot turn back into a literal
// (identical calls are merged).
__device__ __forceinline__ uint32_t magic_pair_reg() {
  uint32_t m;
  asm("v_mov_b32 %0, 0x43004300" : "=v"(m));
  return m;
}

// kNibblePairMask in an SGPR, likewise.
__device__ __forceinline__ uint32_t nibble_mask_reg() {
  uint32_t m;
  asm("s_mov_b32 %0, 0x000f000f" : "=s"(m));
  return m;
}

// Two nibbles of `word` (positions j and j+4, j = shift/4) as bfloat16 (128+q) pair:
// ((word >> shift) & kNibblePairMask) | kMagicPair, one v_and_or_b32 after the
// shift.  A VOP3 instruction on this target takes at most one literal, so both
// constants come from registers; the and-or itself is ordinary code, so the
// compiler sees the register it writes and keeps the wait states a matrix
// instruction reading it needs (an asm-emitted write would hide that).
__device__ __forceinline__ uint32_t nib_pair(uint32_t word, int shift) {
  static_assert(kNibblePairMask == 0x000F000Fu && kMagicPair == 0x43004300u, "constants in the asm above");
  return ((word >> shift) & nibble_mask_reg()) | magic_pair_reg();
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

// ---- cross-lane steps without LDS traffic: DPP inside 16-lane rows, the gfx950
// permlane swaps across rows and halves.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Exchange across the two 16-lane rows of each 32-lane half (row r <-> r^1) and
// across the two 32-lane halves.  Each swap returns the pair {own, other} in an
// order that depends on the lane, so callers combine the pair symmetrically
// (sum, max).
__device__ __forceinline__ void swap_rows16(uint32_t v, uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap_halves32(uint32_t v, uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}

// Sum over aligned groups of 2^lshift consecutive lanes (lshift 0..6, uniform);
// every lane of a group ends with the group total.  The mirror steps are sums
// once both mirrored halves already hold equal partial totals.
__device__ __forceinline__ float group_sum_rt(float v, int lshift) {
  if (lshift >= 1) v += dpp_f32<kDppQuadXor1>(v);
  if (lshift >= 2) v += dpp_f32<kDppQuadXor2>(v);
  if (lshift >= 3) v += dpp_f32<kDppRowHalfMirror>(v);
  if (lshift >= 4) v += dpp_f32<kDppRowMirror>(v);
  uint32_t a, b;
  if (lshift >= 5) { swap_rows16(__float_as_uint(v), a, b); v = __uint_as_float(a) + __uint_as_float(b); }
  if (lshift >= 6) { swap_halves32(__float_as_uint(v), a, b); v = __uint_as_float(a) + __uint_as_float(b); }
  return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
  constexpr int sh = W >= 64 ? 6 : W >= 32 ? 5 : W >= 16 ? 4 : W >= 8 ? 3 : W >= 4 ? 2 : W >= 2 ? 1 : 0;
  return group_sum_rt(v, sh);
}

// Maximum over the whole wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  uint32_t a, b;
  swap_rows16(v, a, b);
  v = max(a, b);
  swap_halves32(v, a, b);
  return max(a, b);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Order-preserving map of a float to uint32 (larger float -> larger key); 0 is
// below every key of a non-NaN float.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// ---- device-coherent data exchange between workgroups of one grid.
// The XCDs' L2 caches are not coherent with each other.  Values handed from one
// workgroup to another inside a kernel are stored and loaded with agent-scope
// atomics (write-through / L2-bypassing accesses), so no L2 writeback or
// invalidation of the whole cache is needed to publish or observe them.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Word 3 of a raw buffer resource (no format conversion, bounds-checked by
// byte count) and the cache-policy bits of a device-scope (sc1) load.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kLoadDeviceScope = 16;

// s_waitcnt immediate for "at most n vector-memory ops outstanding" (gfx9 encoding,
// expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// The same with lgkmcnt(0) (all of this wave's LDS reads done).
constexpr int vmcnt_lgkm0_imm(int n) { return vmcnt_imm(n) & ~(0xF << 8); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses, not
// for its outstanding global loads (a __syncthreads would also wait for those, so
// loads issued ahead of a barrier would have to land before it).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Grid-wide barrier over `nblocks` co-resident workgroups.  State {count, gen}
// lives in caller memory that is zero when first used; count returns to zero
// after every barrier.  Every thread first waits for its own outstanding
// stores, so agent-scope stores issued before the barrier are visible after it.
struct GridBarrier {
  unsigned count;
  unsigned gen;
  unsigned timeouts;  // waits abandoned after kBarrierSpinLimit polls (a misuse: should stay 0)
};

// Each poll is a device-coherent load (about a microsecond), so this bounds a
// wait to roughly a quarter of a second; a corrupted barrier state then costs a
// wrong result and a recorded timeout, not a hang.
constexpr unsigned kBarrierSpinLimit = 1u << 18;

__device__ __forceinline__ void grid_barrier(GridBarrier* bar, unsigned nblocks) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned g = __hip_atomic_load(&bar->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmem();  // the generation is read before this workgroup is counted
    const unsigned arrived = __hip_atomic_fetch_add(&bar->count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (arrived == nblocks - 1) {
      __hip_atomic_store(&bar->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_vmem();  // the reset lands before the release
      __hip_atomic_fetch_add(&bar->gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      unsigned spins = 0;
      while (__hip_atomic_load(&bar->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kBarrierSpinLimit) {
          __hip_atomic_fetch_add(&bar->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    wait_vmem();
  }
  __syncthreads();
}

}  // namespace q4moe
