// Router (logits, softmax top-k, renormalised weights) for a block of tokens,
// and the stable counting sort that groups (token, slot) rows by expert for
// the prefill expert GEMM (lily-qwen3.8-flash-next README, "How the speed was
// achieved": prefill runs the expert GEMM over token-to-expert groups).
#include "kernels.h"
#include "topk.h"

namespace q4moe {

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// logits[t][e] = X[t] . router[e]: bf16 MFMA 32x32x16, fp32 accumulation.
// Workgroup = 2x2 waves = 64 tokens x 64 experts; every lane loads its own
// 64-byte strips of X and router per 64-column step, so both operands use the
// same (arbitrary but consistent) order of the 64 columns inside a step.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ router,
                                                            const uint16_t* __restrict__ X, int64_t T, int E,
                                                            int H, float* __restrict__ logits) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
  const int e0 = blockIdx.y * 64 + (wave >> 1) * 32;
  const int m = lane & 31, h = lane >> 5;
  const int64_t trow = min<int64_t>(t0 + m, T - 1);
  const int erow = min(e0 + m, E - 1);
  const uint4* xa = reinterpret_cast<const uint4*>(X + trow * H) + 4 * h;
  const uint4* rb = reinterpret_cast<const uint4*>(router + (int64_t)erow * H) + 4 * h;
  f32x16_t acc = {};
  for (int k0 = 0; k0 < H; k0 += 64) {
    uint4 av[4], bv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) { av[s] = xa[(k0 >> 3) + s]; bv[s] = rb[(k0 >> 3) + s]; }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[s]),
                                                    __builtin_bit_cast(bf16x8_t, bv[s]), acc, 0, 0, 0);
  }
  // D layout: column (expert) = lane % 32, row (token) = 8*(i/4) + 4*(lane/32) + i%4
  const int e = e0 + m;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t t = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (t < T && e < E) logits[t * E + e] = acc[i];
  }
}

__global__ __launch_bounds__(256) void topk_rows_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ int32_t s_ids[4][kMaxTopK];
  __shared__ float s_w[4][kMaxTopK];
  const int wave = threadIdx.x / kWave;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  wave_topk(logits + t * E, E, k, s_ids[wave], s_w[wave]);
  const int lane = lane_id();
  if (lane < k) {
    ids[t * k + lane] = s_ids[wave][lane];
    weights[t * k + lane] = s_w[wave][lane];
  }
}

// ---- stable counting sort by expert via per-expert row bitmaps
// bitmap[e][w] bit b <=> row 32*w + b has expert e.  The position of row r in
// its segment is the number of set bits before it, so the order inside a
// segment is increasing r (stable) and independent of scheduling.

__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void bitmap_set_kernel(const int32_t* __restrict__ ids, int64_t rows, int E, int64_t W,
                                  uint32_t* __restrict__ bitmap) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += (int64_t)gridDim.x * blockDim.x) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicOr(&bitmap[(int64_t)e * W + (r >> 5)], 1u << (r & 31));
  }
}

// One workgroup per expert: exclusive prefix of popcounts over its W words.
__global__ __launch_bounds__(256) void bitmap_scan_kernel(const uint32_t* __restrict__ bitmap, int64_t W,
                                                          uint32_t* __restrict__ prefix, int32_t* __restrict__ counts) {
  __shared__ int32_t s_part[256];
  const int e = blockIdx.x;
  const uint32_t* bm = bitmap + (int64_t)e * W;
  uint32_t* pre = prefix + (int64_t)e * W;
  const int64_t per = (W + blockDim.x - 1) / blockDim.x;
  const int64_t w0 = threadIdx.x * per, w1 = min<int64_t>(W, w0 + per);
  int32_t local = 0;
  for (int64_t w = w0; w < w1; ++w) local += __popc(bm[w]);
  s_part[threadIdx.x] = local;
  __syncthreads();
  // inclusive Hillis-Steele scan over the 256 partial sums
  for (int off = 1; off < 256; off <<= 1) {
    int32_t v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
    __syncthreads();
    s_part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = s_part[threadIdx.x] - local;
  for (int64_t w = w0; w < w1; ++w) {
    pre[w] = run;
    run += __popc(bm[w]);
  }
  if (threadIdx.x == blockDim.x - 1) counts[e] = s_part[threadIdx.x];
}

// One workgroup: offsets = exclusive scan of counts; tile_offsets likewise of ceil(count/tile_rows).
__global__ __launch_bounds__(1024) void offsets_scan_kernel(const int32_t* __restrict__ counts, int E,
                                                            int32_t* __restrict__ offsets, int tile_rows,
                                                            int32_t* __restrict__ tile_offsets) {
  __shared__ int32_t s_c[1024];
  __shared__ int32_t s_t[1024];
  const int i = threadIdx.x;
  const int32_t c = i < E ? counts[i] : 0;
  const int32_t tc = (tile_rows > 0 && i < E) ? (c + tile_rows - 1) / tile_rows : 0;
  s_c[i] = c;
  s_t[i] = tc;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t a = i >= off ? s_c[i - off] : 0;
    int32_t b = i >= off ? s_t[i - off] : 0;
    __syncthreads();
    s_c[i] += a;
    s_t[i] += b;
    __syncthreads();
  }
  if (i < E) {
    offsets[i + 1] = s_c[i];
    if (tile_offsets) tile_offsets[i + 1] = s_t[i];
  }
  if (i == 0) {
    offsets[0] = 0;
    if (tile_offsets) tile_offsets[0] = 0;
  }
}

__global__ void permute_scatter_kernel(const int32_t* __restrict__ ids, int64_t rows, int E, int64_t W,
                                       const uint32_t* __restrict__ bitmap, const uint32_t* __restrict__ prefix,
                                       const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows,
                                       int32_t* __restrict__ inv_rows) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += (int64_t)gridDim.x * blockDim.x) {
    const int e = ids[r];
    if (e < 0 || e >= E) continue;
    const int64_t w = (int64_t)e * W + (r >> 5);
    const uint32_t below = bitmap[w] & ((1u << (r & 31)) - 1u);
    const int32_t pos = offsets[e] + (int32_t)prefix[w] + __popc(below);
    sorted_rows[pos] = (int32_t)r;
    inv_rows[r] = pos;
  }
}

int grid_for(int64_t n, int block) {
  int64_t b = (n + block - 1) / block;
  if (b > 65536) b = 65536;
  return (int)(b < 1 ? 1 : b);
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int n_experts) { return align256((size_t)T * n_experts * 4); }

hipError_t run_route_topk(const uint16_t* router, int E, int H, const uint16_t* X, int64_t T, int k, int32_t* ids,
                          float* weights, void* ws, hipStream_t stream) {
  float* logits = static_cast<float*>(ws);
  dim3 grid((unsigned)((T + 63) / 64), (unsigned)((E + 63) / 64));
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, router, X, T, E, H, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, logits, T, E, k, ids,
                     weights);
  return hipGetLastError();
}

size_t permute_workspace_bytes(int64_t rows, int n_experts) {
  const int64_t W = (rows + 31) / 32;
  return 2 * align256((size_t)n_experts * W * 4) + align256((size_t)n_experts * 4);
}

hipError_t run_permute(const int32_t* ids, int64_t rows, int E, int32_t* offsets, int32_t* sorted_rows,
                       int32_t* inv_rows, void* ws, int tile_rows, int32_t* tile_offsets, hipStream_t stream) {
  const int64_t W = (rows + 31) / 32;
  char* w = static_cast<char*>(ws);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)E * W * 4);
  uint32_t* prefix = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)E * W * 4);
  int32_t* counts = reinterpret_cast<int32_t*>(w);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(E * W, 256)), dim3(256), 0, stream, bitmap, (int64_t)E * W);
  hipLaunchKernelGGL(bitmap_set_kernel, dim3(grid_for(rows, 256)), dim3(256), 0, stream, ids, rows, E, W, bitmap);
  hipLaunchKernelGGL(bitmap_scan_kernel, dim3(E), dim3(256), 0, stream, bitmap, W, prefix, counts);
  hipLaunchKernelGGL(offsets_scan_kernel, dim3(1), dim3(1024), 0, stream, counts, E, offsets, tile_rows,
                     tile_offsets);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(grid_for(rows, 256)), dim3(256), 0, stream, ids, rows, E, W,
                     bitmap, prefix, offsets, sorted_rows, inv_rows);
  return hipGetLastError();
}

}  // namespace q4moe
