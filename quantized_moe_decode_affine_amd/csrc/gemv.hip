// Batch-1..8 Q4 GEMV: the decode-form weight stream (lily-qwen3.8-flash-next
// README, "How the speed was achieved": a decode step reads every weight
// once and is bandwidth-bound), with an optional fused greedy argmax for the
// LM head (lily README, introduction: decoding is always greedy).
//
// Mapping: L lanes cover one row (L = min(64, groups per row), a power of
// two), each lane takes one 64-column group per step (two uint4 code loads,
// one scale, one bias), so a wave instruction reads 64/L rows of contiguous
// code bytes.  Each lane keeps S rows in flight.  Activations are staged once
// per workgroup in LDS as permuted bfloat16 pairs; the group products run on
// v_dot2 with exact 128+q dequantization (common.h), the row sum is a lane
// butterfly.
#include "kernels.h"
#include "vecstage.h"

namespace q4moe {

namespace {

struct GemvParams {
  const uint4* codes;      // [rows][k/32] as uint4
  const uint16_t* scales;  // [rows][k/64]
  const uint16_t* biases;
  int64_t rows;
  int k;
  int lshift;              // log2 of lanes per row
  const uint16_t* x;       // [B][k]
  void* y;                 // store mode: [B][rows]
  int out_bf16;
  float* part_val;         // argmax mode: [gridDim.x][B]
  int32_t* part_idx;
};

__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi) {
  return v > bv || (v == bv && i < bi);
}

template <int S, int B, bool ARGMAX>
__global__ __launch_bounds__(256) void q4_gemv_kernel(GemvParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  constexpr int ST = chunk_stride<1>();
  const int C = p.k >> 5;
  const int G = p.k >> 6;
  uint32_t* vp = smem;
  float* vs = reinterpret_cast<float*>(smem + B * C * ST);
#pragma unroll
  for (int b = 0; b < B; ++b) stage_bf16_vector(p.x + (size_t)b * p.k, C, vp + b * C * ST, vs + b * C);
  __syncthreads();

  const int lane = lane_id();
  const int L = 1 << p.lshift;
  const int sub = lane & (L - 1);
  const int rsub = lane >> p.lshift;
  const int rpi = kWave >> p.lshift;
  const int wpb = blockDim.x / kWave;
  const int64_t wave = (int64_t)blockIdx.x * wpb + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * wpb;
  const int64_t step = (int64_t)rpi * S;

  float best[B];
  int32_t besti[B];
#pragma unroll
  for (int b = 0; b < B; ++b) { best[b] = -INFINITY; besti[b] = 0x7FFFFFFF; }

  for (int64_t base = wave * step; base < p.rows; base += nwaves * step) {
    float acc[S][B];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[s][b] = 0.f;

    for (int g = sub; g < G; g += L) {
      uint4 c0[S], c1[S];
      uint32_t sb[S], bb[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int64_t row = base + (int64_t)s * rpi + rsub;
        if (row < p.rows) {
          const uint4* cr = p.codes + row * C + 2 * g;
          c0[s] = cr[0];
          c1[s] = cr[1];
          sb[s] = p.scales[row * G + g];
          bb[s] = p.biases[row * G + g];
        } else {
          c0[s] = c1[s] = make_uint4(0, 0, 0, 0);
          sb[s] = bb[s] = 0;
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint32_t* v = vp + b * C * ST + 2 * g * ST;
        const float vsum = vs[b * C + 2 * g] + vs[b * C + 2 * g + 1];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          float pd = chunk_pdot<1>(c0[s], v) + chunk_pdot<1>(c1[s], v + ST);
          acc[s][b] += affine_term(pd, vsum, sb[s], bb[s]);
        }
      }
    }

#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int b = 0; b < B; ++b)
        for (int m = 1; m < L; m <<= 1) acc[s][b] += __shfl_xor(acc[s][b], m, kWave);

#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t row = base + (int64_t)s * rpi + rsub;
      if (row >= p.rows) continue;
      if constexpr (ARGMAX) {
#pragma unroll
        for (int b = 0; b < B; ++b)
          if (better(acc[s][b], (int32_t)row, best[b], besti[b])) { best[b] = acc[s][b]; besti[b] = (int32_t)row; }
      } else if (sub == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.y)[(size_t)b * p.rows + row] = (uint16_t)f32_to_bf16_bits(acc[s][b]);
          else
            reinterpret_cast<float*>(p.y)[(size_t)b * p.rows + row] = acc[s][b];
        }
      }
    }
  }

  if constexpr (ARGMAX) {
    __shared__ float red_v[B][4];
    __shared__ int32_t red_i[B][4];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = best[b];
      int32_t i = besti[b];
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) {
        float ov = __shfl_xor(v, m, kWave);
        int32_t oi = __shfl_xor(i, m, kWave);
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
      }
      if (lane == 0) { red_v[b][threadIdx.x / kWave] = v; red_i[b][threadIdx.x / kWave] = i; }
    }
    __syncthreads();
    if (threadIdx.x < B) {
      const int b = threadIdx.x;
      float v = red_v[b][0];
      int32_t i = red_i[b][0];
      for (int w = 1; w < wpb; ++w)
        if (better(red_v[b][w], red_i[b][w], v, i)) { v = red_v[b][w]; i = red_i[b][w]; }
      p.part_val[(size_t)blockIdx.x * B + b] = v;
      p.part_idx[(size_t)blockIdx.x * B + b] = i;
    }
  }
}

// One workgroup reduces the per-block (value, index) partials of each batch row.
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const float* part_val, const int32_t* part_idx,
                                                              int nparts, int B, int32_t* ids, float* max_logit) {
  __shared__ float sv[4];
  __shared__ int32_t si[4];
  for (int b = 0; b < B; ++b) {
    float v = -INFINITY;
    int32_t i = 0x7FFFFFFF;
    for (int j = threadIdx.x; j < nparts; j += blockDim.x) {
      float ov = part_val[(size_t)j * B + b];
      int32_t oi = part_idx[(size_t)j * B + b];
      if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      float ov = __shfl_xor(v, m, kWave);
      int32_t oi = __shfl_xor(i, m, kWave);
      if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
    if (lane_id() == 0) { sv[threadIdx.x / kWave] = v; si[threadIdx.x / kWave] = i; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = sv[0];
      int32_t bi = si[0];
      for (int w = 1; w < (int)(blockDim.x / kWave); ++w)
        if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
      ids[b] = bi;
      if (max_logit) max_logit[b] = bv;
    }
    __syncthreads();
  }
}

int log2_floor(int64_t v) {
  int r = 0;
  while ((int64_t(1) << (r + 1)) <= v) ++r;
  return r;
}

struct GemvGrid {
  int blocks;
  int lshift;
};

GemvGrid gemv_grid(int64_t rows, int k, int S) {
  const int G = k / kGroup;
  GemvGrid g;
  g.lshift = log2_floor(G < kWave ? G : kWave);
  const int64_t rows_per_wave_iter = (int64_t)(kWave >> g.lshift) * S;
  const int64_t iters = (rows + rows_per_wave_iter - 1) / rows_per_wave_iter;
  int64_t max_waves = (int64_t)device_cu_count() * 16;
  if (max_waves > 8192) max_waves = 8192;  // at most 2048 blocks: bounds the argmax partials
  const int64_t per_wave = (iters + max_waves - 1) / max_waves;
  const int64_t waves = (iters + per_wave - 1) / per_wave;
  g.blocks = (int)((waves + 3) / 4);
  return g;
}

template <int S, int B, bool ARGMAX>
hipError_t launch_gemv(GemvParams p, const GemvGrid& g, hipStream_t stream) {
  const size_t lds = (size_t)B * (p.k / 32) * (chunk_stride<1>() * 4 + 4);
  hipLaunchKernelGGL((q4_gemv_kernel<S, B, ARGMAX>), dim3(g.blocks), dim3(256), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t gemv_lds_bytes(int k, int B) { return (size_t)B * (k / 32) * (chunk_stride<1>() * 4 + 4); }

int lmhead_partial_blocks(int64_t rows, int k, int B) {
  const int S = B <= 2 ? 4 : (B <= 4 ? 2 : 1);
  return gemv_grid(rows, k, S).blocks;
}

hipError_t run_q4_gemv(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
                       int k, const uint16_t* x, void* y, int out_bf16, hipStream_t stream) {
  GemvParams p{};
  p.codes = reinterpret_cast<const uint4*>(codes);
  p.scales = scales;
  p.biases = biases;
  p.rows = rows;
  p.k = k;
  p.x = x;
  p.y = y;
  p.out_bf16 = out_bf16;
  GemvGrid g = gemv_grid(rows, k, 4);
  p.lshift = g.lshift;
  return launch_gemv<4, 1, false>(p, g, stream);
}

hipError_t run_lmhead_argmax(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                             int64_t rows, int k, const uint16_t* X, int B, int32_t* ids, float* max_logit,
                             float* part_val, int32_t* part_idx, hipStream_t stream) {
  GemvParams p{};
  p.codes = reinterpret_cast<const uint4*>(codes);
  p.scales = scales;
  p.biases = biases;
  p.rows = rows;
  p.k = k;
  p.x = X;
  p.part_val = part_val;
  p.part_idx = part_idx;
  const int S = B <= 2 ? 4 : (B <= 4 ? 2 : 1);
  GemvGrid g = gemv_grid(rows, k, S);
  p.lshift = g.lshift;
  hipError_t e;
  switch (B) {
    case 1: e = launch_gemv<4, 1, true>(p, g, stream); break;
    case 2: e = launch_gemv<4, 2, true>(p, g, stream); break;
    case 3: e = launch_gemv<2, 3, true>(p, g, stream); break;
    case 4: e = launch_gemv<2, 4, true>(p, g, stream); break;
    case 5: e = launch_gemv<1, 5, true>(p, g, stream); break;
    case 6: e = launch_gemv<1, 6, true>(p, g, stream); break;
    case 7: e = launch_gemv<1, 7, true>(p, g, stream); break;
    case 8: e = launch_gemv<1, 8, true>(p, g, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(1), dim3(256), 0, stream, part_val, part_idx, g.blocks, B,
                     ids, max_logit);
  return hipGetLastError();
}

}  // namespace q4moe
