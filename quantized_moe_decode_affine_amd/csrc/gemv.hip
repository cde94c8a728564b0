// Batch-1..8 Q4 GEMV: the decode-form weight stream (lily-qwen3.8-flash-next
// README, "How the speed was achieved": a decode step reads every weight
// once and is bandwidth-bound), with an optional fused greedy argmax for the
// LM head (lily README, introduction: decoding is always greedy).
//
// Mapping: L lanes cover one row (L = min(64, groups per row), a power of
// two), each lane takes one 64-column group per step (two uint4 code loads,
// one scale, one bias), so a wave instruction reads 64/L rows of contiguous
// code bytes.  Each lane keeps S rows in flight, and where a lane owns exactly
// one group per row the next step's rows are loaded while the current one
// computes.  Activations are staged once per workgroup in LDS as permuted
// bfloat16 pairs; the group products run on v_dot2 with exact 128+q
// dequantization (common.h), the row sums are DPP/permlane reductions.
#include <mutex>

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
  int chunk_lanes;         // 1: exactly one group per lane (lanes per row == k/64)
  const uint16_t* x;       // [B][k]
  void* y;                 // store mode: [B][rows]
  int out_bf16;
  unsigned long long* keys;  // argmax mode: [B] running {value key : ~index} maxima (0 between calls)
  unsigned* done;          // argmax mode: arrival counter (0 between calls)
  int32_t* ids;            // argmax mode: [B]
  float* max_logit;        // argmax mode: [B] or null
};

__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi) {
  return v > bv || (v == bv && i < bi);
}

// Greedy argmax over a grid: every lane passes its running (max, lowest index)
// per batch row (-inf and index 0x7FFFFFFF for rows it does not hold).  The pair
// is one 64-bit key, {order-preserving key of the value : ~index}, so the largest
// key is the largest value with the lowest index.  A wave reduces the keys with
// two DPP maxima (value keys, then the inverted indices of the lanes holding the
// largest), the workgroup folds its waves in LDS and applies one 64-bit atomic max
// per batch row to keys[b]; the last workgroup to arrive reads the keys, writes
// ids and max_logit, and leaves keys and the arrival counter at zero for the next
// call.
template <int B>
__device__ __forceinline__ void argmax_epilogue(float (&best)[B], int32_t (&besti)[B], const GemvParams& p) {
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  __shared__ uint32_t red_hi[B][4], red_lo[B][4];
  __shared__ int s_last;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const uint32_t hi = float_key(best[b]);
    const uint32_t m = wave_max_u32(hi);
    const uint32_t lo = wave_max_u32(hi == m ? ~(uint32_t)besti[b] : 0u);
    if (lane == 0) { red_hi[b][threadIdx.x / kWave] = m; red_lo[b][threadIdx.x / kWave] = lo; }
  }
  __syncthreads();
  if (threadIdx.x < B) {
    const int b = threadIdx.x;
    unsigned long long key = 0;
    for (int w = 0; w < wpb; ++w) {
      const unsigned long long kw = (unsigned long long)red_hi[b][w] << 32 | red_lo[b][w];
      key = kw > key ? kw : key;
    }
    __hip_atomic_fetch_max(p.keys + b, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_vmem();  // this thread's atomic max has been performed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (s_last && threadIdx.x < B) {
    const int b = threadIdx.x;
    const unsigned long long key = __hip_atomic_load(p.keys + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p.ids[b] = (int32_t)~(uint32_t)key;
    if (p.max_logit) p.max_logit[b] = key_float((uint32_t)(key >> 32));
    __hip_atomic_store(p.keys + b, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (s_last && threadIdx.x == 0) __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int S, int B, bool ARGMAX, bool CHUNK>
__global__ __launch_bounds__(256) void q4_gemv_kernel(GemvParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  constexpr int ST = chunk_stride<1>();
  const int C = p.k >> 5;
  const int G = p.k >> 6;
  uint32_t* vp = smem;
  float* vs = reinterpret_cast<float*>(smem + B * C * ST);
  // One batch row in chunks of one thread each: the thread's 64 bytes of x are loaded
  // now (past the last chunk, the last one again) and staged after the first rows'
  // loads are out, so the two latencies overlap.
  const bool xpre = CHUNK && B == 1 && C <= (int)blockDim.x;
  uint4 xw[4];
  if (xpre) {
    const uint4* src = reinterpret_cast<const uint4*>(p.x) + 4 * min((int)threadIdx.x, C - 1);
#pragma unroll
    for (int b = 0; b < 4; ++b) xw[b] = src[b];
  } else {
#pragma unroll
    for (int b = 0; b < B; ++b) stage_bf16_vector(p.x + (size_t)b * p.k, C, vp + b * C * ST, vs + b * C);
    __syncthreads();
  }

  const int lane = lane_id();
  const int L = 1 << p.lshift;
  const int sub = lane & (L - 1);
  const int rsub = lane >> p.lshift;
  const int rpi = kWave >> p.lshift;
  const int wpb = blockDim.x / kWave;
  const int64_t wave = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
  const int64_t nwaves = (int64_t)gridDim.x * wpb;
  const int64_t step = (int64_t)rpi * S;

  float best[B];
  int32_t besti[B];
#pragma unroll
  for (int b = 0; b < B; ++b) { best[b] = -INFINITY; besti[b] = 0x7FFFFFFF; }

  // Row totals of one step (every lane of a row's group holds them): store, or
  // fold into this lane's running argmax.
  auto emit = [&](int64_t base, float (&acc)[S][B]) __attribute__((always_inline)) {
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
  };

  if constexpr (CHUNK) {
    // One lane per 64-column group of a row (L == G): the group's activation
    // pairs and sum are loop invariants (in registers for B <= 2); each row's
    // codes are converted once and shared by the batch rows; row sums are
    // DPP/permlane reductions over the row's L lanes.
    constexpr bool kXReg = B <= 2;
    const int g = sub;
    float vsum[B];
    uint32_t xr[kXReg ? B : 1][32];
    struct RowFrag {
      uint4 c0, c1;
      uint32_t s, b;
    };
    auto convert = [&](const RowFrag& f, uint32_t (&q)[32]) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const uint4& u = w < 4 ? f.c0 : f.c1;
        const uint32_t word = (w & 3) == 0 ? u.x : (w & 3) == 1 ? u.y : (w & 3) == 2 ? u.z : u.w;
#pragma unroll
        for (int j = 0; j < 4; ++j) q[4 * w + j] = nib_pair(word, 4 * j);
      }
    };
    auto dot = [&](const uint32_t (&q)[32], const uint32_t* xv) __attribute__((always_inline)) {
      float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
      for (int j = 0; j < 32; j += 4) {
        p0 = dot2_bf16(q[j], xv[j], p0);
        p1 = dot2_bf16(q[j + 1], xv[j + 1], p1);
        p2 = dot2_bf16(q[j + 2], xv[j + 2], p2);
        p3 = dot2_bf16(q[j + 3], xv[j + 3], p3);
      }
      return (p0 + p1) + (p2 + p3);
    };
    // The rows of step base (S per lane), loaded into registers.  Bases past the end
    // read the last row (in bounds, unused), so every step issues the same loads.
    auto load_step = [&](int64_t base, RowFrag (&f)[S]) __attribute__((always_inline)) {
      base = min<int64_t>(base, p.rows - 1);
      // uniform 64-bit step bases, small 32-bit row offsets inside the step
      const uint4* cb = p.codes + base * C;
      const uint16_t* sp = p.scales + base * G;
      const uint16_t* bp = p.biases + base * G;
      const int left = (int)min<int64_t>(p.rows - 1 - base, (int64_t)S * rpi);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int r = min(s * rpi + rsub, left);  // rows past the end: loaded, unused
        f[s].c0 = cb[r * C + 2 * g];
        f[s].c1 = cb[r * C + 2 * g + 1];
        f[s].s = sp[r * G + g];
        f[s].b = bp[r * G + g];
      }
    };
    // Software-pipelined over two register sets: the next step's rows are in flight
    // while this step computes (the sets swap roles, so no copy waits for the loads).
    auto compute_step = [&](int64_t base, const RowFrag (&F)[S]) __attribute__((always_inline)) {
      float acc[S][B];
      if constexpr (kXReg) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          __builtin_amdgcn_sched_barrier(0);  // one row at a time: a row's converted codes take 32 registers
          uint32_t q[32];
          convert(F[s], q);
#pragma unroll
          for (int b = 0; b < B; ++b) acc[s][b] = affine_term(dot(q, xr[b]), vsum[b], F[s].s, F[s].b);
        }
      } else {
        uint32_t q[S][32];
#pragma unroll
        for (int s = 0; s < S; ++s) convert(F[s], q[s]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          uint32_t xl[32];
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) {
            const uint4 t = *reinterpret_cast<const uint4*>(vp + b * C * ST + (2 * g + (qq >> 2)) * ST + 4 * (qq & 3));
            xl[4 * qq] = t.x;
            xl[4 * qq + 1] = t.y;
            xl[4 * qq + 2] = t.z;
            xl[4 * qq + 3] = t.w;
          }
#pragma unroll
          for (int s = 0; s < S; ++s) acc[s][b] = affine_term(dot(q[s], xl), vsum[b], F[s].s, F[s].b);
        }
      }
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[s][b] = group_sum_rt(acc[s][b], p.lshift);
      emit(base, acc);
    };
    const int64_t stride = nwaves * step;
    RowFrag fa[S], fb[S];
    load_step(wave * step, fa);
    if (xpre) {
      if ((int)threadIdx.x < C) {
        float sx = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint4 v = xw[b];
          sx += (bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16)) +
                (bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16)) +
                (bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16)) +
                (bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16));
          *reinterpret_cast<uint4*>(vp + threadIdx.x * ST + 4 * b) = permute_block(v);
        }
        vs[threadIdx.x] = sx;
      }
      lds_sync();  // (the first rows' loads stay in flight)
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      vsum[b] = vs[b * C + 2 * g] + vs[b * C + 2 * g + 1];
      if constexpr (kXReg) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint4 t = *reinterpret_cast<const uint4*>(vp + b * C * ST + (2 * g + (q >> 2)) * ST + 4 * (q & 3));
          xr[b][4 * q] = t.x;
          xr[b][4 * q + 1] = t.y;
          xr[b][4 * q + 2] = t.z;
          xr[b][4 * q + 3] = t.w;
        }
      }
    }
    for (int64_t base = wave * step; base < p.rows; base += 2 * stride) {
      // keeps the (loop-invariant) LDS activation reads of B > 2 inside the loop:
      // hoisted, they would hold 32 registers per batch row
      if constexpr (!kXReg) asm volatile("" ::: "memory");
      load_step(base + stride, fb);
      compute_step(base, fa);
      if (base + stride >= p.rows) break;
      load_step(base + 2 * stride, fa);
      compute_step(base + stride, fb);
    }
  } else {
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
        for (int b = 0; b < B; ++b) acc[s][b] = group_sum_rt(acc[s][b], p.lshift);
      emit(base, acc);
    }
  }

  if constexpr (ARGMAX) argmax_epilogue<B>(best, besti, p);
}


// Batch-1..7 GEMV over 8-bit affine codes (the 8-bit exceptions of the checkpoint:
// lily-qwen3.8-flash-next README, "The model": the q4-xl conversion keeps the LM head
// and the shared expert at 8 bits; "2026-09-02: Lily vs MLX 0.32.2", "Hardware and
// software": affine Q8 router-gate exceptions).  Code j of a row is byte j%4 of word
// j/4; w = scale*q + bias per 64-column group.  The activations are staged once per
// workgroup in LDS as fp32 with their per-group sums, the groups interleaved by 4-value
// chunks (chunk c of group g at (c*G + g)*4) so that the lanes of a row, each on its own
// group, read consecutive 16-byte words; a lane takes one group of a row
// at a time (64 code bytes: four 16-byte loads), converts each byte to fp32 (exact),
// and accumulates the exact 8-bit x 8-bit products in fp32: per group
// scale * sum(x q) + bias * sum(x).  Rows are strided over the waves as in the
// 4-bit kernel, S rows per lane in flight; the L lanes of a row reduce with DPP.
template <int S, int B, bool ARGMAX>
__global__ __launch_bounds__(256) void q8_gemv_kernel(GemvParams p) {
  extern __shared__ __align__(16) float q8_smem[];
  const int K = p.k, G = K >> 6, C16 = K >> 4;  // C16: 16-byte code chunks per row
  float* xs = q8_smem;             // [B][16 chunks][G][4]
  float* gs = q8_smem + B * K;     // [B][G]
  auto xslot = [&](int b, int g, int j) { return b * K + ((j >> 2) * G + g) * 4 + (j & 3); };
  for (int i = threadIdx.x; i < B * K; i += blockDim.x) {
    const int b = i / K, c = i - b * K;
    xs[xslot(b, c >> 6, c & 63)] = bf16_bits_to_f32(p.x[i]);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B * G; i += blockDim.x) {
    const int b = i / G, g = i - b * G;
    float t = 0.f;
    for (int j = 0; j < kGroup; ++j) t += xs[xslot(b, g, j)];  // fixed order
    gs[i] = t;
  }
  __syncthreads();

  const int lane = lane_id();
  const int L = 1 << p.lshift;
  const int sub = lane & (L - 1);
  const int rsub = lane >> p.lshift;
  const int rpi = kWave >> p.lshift;
  const int wpb = blockDim.x / kWave;
  const int64_t wave = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
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
      uint4 c[S][4];
      float sc[S], bi[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int64_t row = min(base + (int64_t)s * rpi + rsub, p.rows - 1);  // past the end: loaded, unused
        const uint4* cr = p.codes + row * C16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) c[s][i] = cr[i];
        sc[s] = bf16_bits_to_f32(p.scales[row * G + g]);
        bi[s] = bf16_bits_to_f32(p.biases[row * G + g]);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float4* xv = reinterpret_cast<const float4*>(xs + b * K) + g;  // chunk c at xv[c * G]
        float P[S];
#pragma unroll
        for (int s = 0; s < S; ++s) P[s] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float4 x4 = xv[(4 * i + w) * G];
#pragma unroll
            for (int s = 0; s < S; ++s) {
              const uint32_t word = w == 0 ? c[s][i].x : w == 1 ? c[s][i].y : w == 2 ? c[s][i].z : c[s][i].w;
              P[s] = fmaf(x4.x, (float)(word & 0xFFu), P[s]);
              P[s] = fmaf(x4.y, (float)((word >> 8) & 0xFFu), P[s]);
              P[s] = fmaf(x4.z, (float)((word >> 16) & 0xFFu), P[s]);
              P[s] = fmaf(x4.w, (float)(word >> 24), P[s]);
            }
          }
        }
        const float xsum = gs[b * G + g];
#pragma unroll
        for (int s = 0; s < S; ++s) acc[s][b] += fmaf(sc[s], P[s], bi[s] * xsum);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t row = base + (int64_t)s * rpi + rsub;
#pragma unroll
      for (int b = 0; b < B; ++b) acc[s][b] = group_sum_rt(acc[s][b], p.lshift);
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
  if constexpr (ARGMAX) argmax_epilogue<B>(best, besti, p);
}

typedef short mfma4_bf16_t __attribute__((ext_vector_type(4)));

// Broadcast of quad lane I's value to its whole quad (DPP quad_perm [I,I,I,I]).
template <int I>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, I * 0x55, 0xF, 0xF, false);
}

// LM head for 2..8 batch rows on the 4x4x4 bf16 MFMA (16 independent 4x4
// blocks per wave instruction).  A wave works through 8-row blocks of the matrix
// (blocks wave, wave + nwaves, ...), each in steps of 8 K groups: block b =
// 8*rq + ks of an instruction covers rows base + 4*rq .. +3 (rq = 0, 1) and K group
// 8*step + ks, with lane 4b+i supplying row i's codes of that group (the 8 blocks
// of a row quad read 256 contiguous bytes of each row), lane 4b+j the activations
// of batch row j (+4 for the second instruction set when B > 4), and lane 4b+j
// receiving the 4 rows' sums for batch row j.  Per group a lane converts 8 code
// words once (exact 128+q pairs, common.h) into 16 A operands, runs 16 MFMAs per
// set into a fresh partial sum P (exact products, fp32 sums) and adds
// s*P + (b - 128 s)*sum_x with its quad's scales and offsets broadcast by DPP; at
// a block's last step the eight groups' sums of a row meet in one lane.  The wave's
// (block, step) items form one stream: the codes of the next two items are in
// flight while the current one computes, across block boundaries, in three
// register sets that take turns (a copy between sets would wait for the loads).
template <int B>
__global__ __launch_bounds__(256) void lmhead_mfma_kernel(GemvParams p) {
  constexpr int NB = (B + 3) / 4;
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
  const int q = lane & 3;          // row of the block (A side) and batch column (B and D sides)
  const int ks = (lane >> 2) & 7;  // group offset of the block
  const int rq = lane >> 5;        // row quad of the block
  int jb[NB];                      // this lane's batch row per set (clamped: columns past B are computed, unused)
#pragma unroll
  for (int h = 0; h < NB; ++h) jb[h] = min(4 * h + q, B - 1);
  const int64_t wave =
      (int64_t)blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  constexpr int kRowsPerBlock = 8;
  const int64_t nblocks = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int spb = (G + 7) >> 3;  // steps per block
  const int64_t my_blocks = wave < nblocks ? (nblocks - 1 - wave) / nwaves + 1 : 0;
  const int64_t n_items = my_blocks * spb;

  float best[NB];
  int32_t besti[NB];
#pragma unroll
  for (int h = 0; h < NB; ++h) { best[h] = -INFINITY; besti[h] = 0x7FFFFFFF; }

  struct Frag {
    uint4 c0, c1;
    uint32_t s, b;
  };
  // Item cursor: block j of the wave and step gs inside it.
  struct Cursor {
    int64_t j;
    int gs;
  };
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.gs == spb) { c.gs = 0; ++c.j; }
  };
  // Loads of the item at c (past the wave's last item, its last block's rows and groups
  // again: in bounds, unused).
  auto load = [&](const Cursor& c) __attribute__((always_inline)) {
    const int64_t jj = min(c.j, my_blocks > 0 ? my_blocks - 1 : 0);
    const int64_t row = min((wave + jj * nwaves) * kRowsPerBlock + 4 * rq + q, p.rows - 1);
    const int g = min(8 * c.gs + ks, G - 1);
    const uint4* cr = p.codes + row * C;
    return Frag{cr[2 * g], cr[2 * g + 1], p.scales[row * G + g], p.biases[row * G + g]};
  };
  f32x4_t acc[NB];
#pragma unroll
  for (int h = 0; h < NB; ++h) acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // One item: its group's products into acc; at the block's last step the row sums.
  auto compute = [&](const Cursor& c, const Frag& f) __attribute__((always_inline)) {
    const int g0 = 8 * c.gs + ks;
    const bool live = g0 < G;  // groups past the end: loaded (clamped), not added
    const int g = min(g0, G - 1);
    uint32_t pr[32];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint4& u = w < 4 ? f.c0 : f.c1;
      const uint32_t word = (w & 3) == 0 ? u.x : (w & 3) == 1 ? u.y : (w & 3) == 2 ? u.z : u.w;
#pragma unroll
      for (int j = 0; j < 4; ++j) pr[4 * w + j] = nib_pair(word, 4 * j);
    }
    const uint32_t s4[4] = {quad_bcast<0>(f.s), quad_bcast<1>(f.s), quad_bcast<2>(f.s), quad_bcast<3>(f.s)};
    const uint32_t b4[4] = {quad_bcast<0>(f.b), quad_bcast<1>(f.b), quad_bcast<2>(f.b), quad_bcast<3>(f.b)};
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      // pair word m of group g sits in chunk 2g + m/16 at offset m%16
      const uint32_t* xv = vp + jb[h] * C * ST + 2 * g * ST;
      f32x4_t P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int m = 2 * t;
        const uint2 xa = *reinterpret_cast<const uint2*>(xv + (m >> 4) * ST + (m & 15));
        P = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(mfma4_bf16_t, make_uint2(pr[m], pr[m + 1])),
                                                 __builtin_bit_cast(mfma4_bf16_t, xa), P, 0, 0, 0);
      }
      const float vsum = vs[jb[h] * C + 2 * g] + vs[jb[h] * C + 2 * g + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] += live ? affine_term(P[i], vsum, s4[i], b4[i]) : 0.f;
    }
    if (c.gs == spb - 1) {
      // the eight group offsets of a row quad meet in the ks = 0 lanes; lane 32rq + j
      // then holds rows base + 4rq + i (i = 0..3) for batch row 4h + j
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[h][i] += __shfl_xor(acc[h][i], 4, kWave);
          acc[h][i] += __shfl_xor(acc[h][i], 8, kWave);
          acc[h][i] += __shfl_xor(acc[h][i], 16, kWave);
        }
      if (ks == 0) {
        const int64_t base = (wave + c.j * nwaves) * kRowsPerBlock;
#pragma unroll
        for (int h = 0; h < NB; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t r = base + 4 * rq + i;
            if (r < p.rows && better(acc[h][i], (int32_t)r, best[h], besti[h])) {
              best[h] = acc[h][i];
              besti[h] = (int32_t)r;
            }
          }
      }
#pragma unroll
      for (int h = 0; h < NB; ++h) acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Item i lives in register set i mod 3; step t loads item t + 2 and computes item
  // t.  The stream starts two steps early (no loads before the loop), so the loop is
  // entered with nothing in flight and the sets rotate without copies.
  Cursor cl{0, 0}, cc{0, 0};  // next item to load, next item to compute
  Frag fa{}, fb{}, fc{};
  for (int64_t t = -2; t < n_items; t += 3) {
    fa = load(cl);
    advance(cl);
    if (t >= 0) {
      compute(cc, fb);
      advance(cc);
    }
    fb = load(cl);
    advance(cl);
    if (t + 1 >= 0 && t + 1 < n_items) {
      compute(cc, fc);
      advance(cc);
    }
    fc = load(cl);
    advance(cl);
    if (t + 2 < n_items) {
      compute(cc, fa);
      advance(cc);
    }
  }
  // every lane offers its candidate for the batch rows it holds, -inf for the others
  float bv[B];
  int32_t bi[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const bool mine = (b & 3) == q;
    bv[b] = mine ? best[b >> 2] : -INFINITY;
    bi[b] = mine ? besti[b >> 2] : 0x7FFFFFFF;
  }
  argmax_epilogue<B>(bv, bi, p);
}

// The same on 8-bit codes (64 bytes per group): pair word m = 4w + j takes bytes j
// of code words 2w and 2w + 1 (columns 8w + j and 8w + j + 4, the staged pair
// order), each exact in bfloat16 as the high half of its fp32 value, and a group
// adds s*P + b*sum_x.
template <int B>
__global__ __launch_bounds__(256) void lmhead_mfma_q8_kernel(GemvParams p) {
  constexpr int NB = (B + 3) / 4;
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
  const int q = lane & 3;          // row of the block (A side) and batch column (B and D sides)
  const int ks = (lane >> 2) & 3;  // group offset of the block
  const int rq = lane >> 4;        // row quad of the block
  int jb[NB];                      // this lane's batch row per set (clamped: columns past B are computed, unused)
#pragma unroll
  for (int h = 0; h < NB; ++h) jb[h] = min(4 * h + q, B - 1);
  const int64_t wave =
      (int64_t)blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  constexpr int kRowsPerWave = 16;

  float best[NB];
  int32_t besti[NB];
#pragma unroll
  for (int h = 0; h < NB; ++h) { best[h] = -INFINITY; besti[h] = 0x7FFFFFFF; }

  constexpr int NC = 4;  // 16-byte code pieces per group
  struct Frag {
    uint4 c[NC];
    uint32_t s, b;
  };
  for (int64_t base = wave * kRowsPerWave; base < p.rows; base += nwaves * kRowsPerWave) {
    const int64_t row = min(base + 4 * rq + q, p.rows - 1);  // rows past the end: loaded, unused
    const uint4* cr = p.codes + row * (NC * G);
    const uint16_t* sr = p.scales + row * G;
    const uint16_t* br = p.biases + row * G;
    f32x4_t acc[NB];
#pragma unroll
    for (int h = 0; h < NB; ++h) acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int g = min(ks, G - 1);
    const int g1 = min(4 + ks, G - 1);
    auto load = [&](int gi) __attribute__((always_inline)) {
      Frag r;
#pragma unroll
      for (int i = 0; i < NC; ++i) r.c[i] = cr[NC * gi + i];
      r.s = sr[gi];
      r.b = br[gi];
      return r;
    };
    Frag f = load(g);
    Frag f1 = load(g1);
    for (int gg = 0; gg < G; gg += 4) {
      const bool live = gg + ks < G;  // groups past the end: loaded (clamped), not added
      const int gn = min(gg + 4 + ks, G - 1);
      const int g2 = min(gg + 8 + ks, G - 1);
      const Frag f2 = load(g2);  // two steps ahead
      uint32_t pr[32];
      uint32_t W[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        W[4 * i] = f.c[i].x;
        W[4 * i + 1] = f.c[i].y;
        W[4 * i + 2] = f.c[i].z;
        W[4 * i + 3] = f.c[i].w;
      }
#pragma unroll
      for (int w = 0; w < 8; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = __float_as_uint((float)((W[2 * w] >> (8 * j)) & 0xFFu)) >> 16;
          const uint32_t hi = __float_as_uint((float)((W[2 * w + 1] >> (8 * j)) & 0xFFu)) & 0xFFFF0000u;
          pr[4 * w + j] = lo | hi;
        }
      const uint32_t s4[4] = {quad_bcast<0>(f.s), quad_bcast<1>(f.s), quad_bcast<2>(f.s), quad_bcast<3>(f.s)};
      const uint32_t b4[4] = {quad_bcast<0>(f.b), quad_bcast<1>(f.b), quad_bcast<2>(f.b), quad_bcast<3>(f.b)};
#pragma unroll
      for (int h = 0; h < NB; ++h) {
        // pair word m of group g sits in chunk 2g + m/16 at offset m%16
        const uint32_t* xv = vp + jb[h] * C * ST + 2 * g * ST;
        f32x4_t P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int m = 2 * t;
          const uint2 xa = *reinterpret_cast<const uint2*>(xv + (m >> 4) * ST + (m & 15));
          P = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(mfma4_bf16_t, make_uint2(pr[m], pr[m + 1])),
                                                   __builtin_bit_cast(mfma4_bf16_t, xa), P, 0, 0, 0);
        }
        const float vsum = vs[jb[h] * C + 2 * g] + vs[jb[h] * C + 2 * g + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float t = fmaf(bf16_bits_to_f32(s4[i]), P[i], bf16_bits_to_f32(b4[i]) * vsum);
          acc[h][i] += live ? t : 0.f;
        }
      }
      f = f1;
      f1 = f2;
      g = gn;
    }
    // the four group offsets of a row quad meet in the ks = 0 lanes; lane 16rq + j
    // then holds rows base + 4rq + i (i = 0..3) for batch row 4h + j
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[h][i] += __shfl_xor(acc[h][i], 4, kWave);
        acc[h][i] += __shfl_xor(acc[h][i], 8, kWave);
      }
    if (ks == 0) {
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = base + 4 * rq + i;
          if (r < p.rows && better(acc[h][i], (int32_t)r, best[h], besti[h])) {
            best[h] = acc[h][i];
            besti[h] = (int32_t)r;
          }
        }
    }
  }
  // every lane offers its candidate for the batch rows it holds, -inf for the others
  float bv[B];
  int32_t bi[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const bool mine = (b & 3) == q;
    bv[b] = mine ? best[b >> 2] : -INFINITY;
    bi[b] = mine ? besti[b >> 2] : 0x7FFFFFFF;
  }
  argmax_epilogue<B>(bv, bi, p);
}

int log2_floor(int64_t v) {
  int r = 0;
  while ((int64_t(1) << (r + 1)) <= v) ++r;
  return r;
}

struct GemvGrid {
  int blocks;
  int lshift;
  int chunk_lanes;
};

// Lanes per row: one per 64-column group; the loop-invariant fast path applies
// when the groups of a row are a power of two, at most 64.
// The grid holds at most one resident round of workgroups (`resident` per CU,
// from the occupancy of the instantiation that will run), so no workgroup
// waits for another to finish; waves stride over the rows.
GemvGrid gemv_grid(int64_t rows, int k, int S, int resident) {
  const int G = k / kGroup;
  GemvGrid g;
  g.chunk_lanes = G <= kWave && (G & (G - 1)) == 0;
  g.lshift = log2_floor(G < kWave ? G : kWave);
  const int64_t rows_per_wave_iter = (int64_t)(kWave >> g.lshift) * S;
  const int64_t iters = (rows + rows_per_wave_iter - 1) / rows_per_wave_iter;
  int64_t max_blocks = (int64_t)device_cu_count() * (resident > 0 ? resident : 1);
  if (max_blocks > kMaxGemvBlocks) max_blocks = kMaxGemvBlocks;  // one resident round at most
  const int64_t blocks = (iters + 3) / 4;
  g.blocks = (int)(blocks < max_blocks ? blocks : max_blocks);
  return g;
}

template <int S, int B, bool ARGMAX, bool CHUNK>
int resident_blocks(size_t lds) {
  static int cached = -1;  // per instantiation; the LDS size only matters for large batches
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, q4_gemv_kernel<S, B, ARGMAX, CHUNK>, 256, lds) != hipSuccess ||
        n < 1)
      n = 1;
    cached = n;
  }
  return cached;
}

size_t gemv_lds(int k, int B) { return (size_t)B * (k / 32) * (chunk_stride<1>() * 4 + 4); }

template <int S, int B, bool ARGMAX>
GemvGrid plan_gemv(int64_t rows, int k) {
  const GemvGrid probe = gemv_grid(rows, k, S, 1);
  const int res = probe.chunk_lanes ? resident_blocks<S, B, ARGMAX, true>(gemv_lds(k, B))
                                    : resident_blocks<S, B, ARGMAX, false>(gemv_lds(k, B));
  return gemv_grid(rows, k, S, res);
}

template <int S, int B, bool ARGMAX>
hipError_t launch_gemv(GemvParams p, const GemvGrid& g, hipStream_t stream) {
  const size_t lds = gemv_lds(p.k, B);
  if (g.chunk_lanes)
    hipLaunchKernelGGL((q4_gemv_kernel<S, B, ARGMAX, true>), dim3(g.blocks), dim3(256), lds, stream, p);
  else
    hipLaunchKernelGGL((q4_gemv_kernel<S, B, ARGMAX, false>), dim3(g.blocks), dim3(256), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t gemv_lds_bytes(int k, int B) { return gemv_lds(k, B); }

namespace {

// Rows per lane and step by batch size (B = 1: two rows, software-pipelined; measured against
// one, four and eight, two leaves the most waves per SIMD with enough bytes in flight).
#ifndef Q4MOE_LMHEAD_ROWS_B1
#define Q4MOE_LMHEAD_ROWS_B1 2
#endif
template <int B>
constexpr int lmhead_rows_per_lane() { return B <= 2 ? Q4MOE_LMHEAD_ROWS_B1 : B <= 4 ? 2 : 1; }

// Workgroups of the head resident per CU at `lds` bytes of LDS each (the activations'
// size grows with k): kept for the last LDS size asked about, asked again when it changes.
template <int B, bool kQ8 = false>
int lmhead_mfma_resident(size_t lds) {
  static std::mutex mu;
  static size_t cached_lds = 0;
  static int cached = -1;
  std::lock_guard<std::mutex> lock(mu);
  if (cached < 0 || cached_lds != lds) {
    int n = 0;
    hipError_t e;
    if constexpr (kQ8)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lmhead_mfma_q8_kernel<B>, 256, lds);
    else
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lmhead_mfma_kernel<B>, 256, lds);
    if (e != hipSuccess || n < 1)
      n = 1;
    cached = n;
    cached_lds = lds;
  }
  return cached;
}

template <int B>
hipError_t run_lmhead_b(GemvParams p, int32_t* ids, float* max_logit, hipStream_t stream) {
  if constexpr (B >= 2) {
    // 8-row blocks over the waves; one resident round of workgroups
    const size_t lds = gemv_lds(p.k, B);
    const int64_t row_blocks = (p.rows + 7) / 8;
    int64_t blocks = (row_blocks + 3) / 4;
    int64_t max_blocks = (int64_t)device_cu_count() * lmhead_mfma_resident<B>(lds);
    if (max_blocks > kMaxGemvBlocks) max_blocks = kMaxGemvBlocks;  // one resident round at most
    if (blocks > max_blocks) blocks = max_blocks;
    p.ids = ids;
    p.max_logit = max_logit;
    hipLaunchKernelGGL((lmhead_mfma_kernel<B>), dim3((int)blocks), dim3(256), lds, stream, p);
    return hipGetLastError();
  }
  constexpr int S = lmhead_rows_per_lane<B>();
  const GemvGrid g = plan_gemv<S, B, true>(p.rows, p.k);
  p.lshift = g.lshift;
  p.chunk_lanes = g.chunk_lanes;
  p.ids = ids;
  p.max_logit = max_logit;
  return launch_gemv<S, B, true>(p, g, stream);
}

}  // namespace

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
  const GemvGrid g = plan_gemv<4, 1, false>(rows, k);
  p.lshift = g.lshift;
  p.chunk_lanes = g.chunk_lanes;
  return launch_gemv<4, 1, false>(p, g, stream);
}

hipError_t run_lmhead_argmax(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                             int64_t rows, int k, const uint16_t* X, int B, int32_t* ids, float* max_logit,
                             unsigned long long* keys, unsigned* done, hipStream_t stream) {
  GemvParams p{};
  p.codes = reinterpret_cast<const uint4*>(codes);
  p.scales = scales;
  p.biases = biases;
  p.rows = rows;
  p.k = k;
  p.x = X;
  p.keys = keys;
  p.done = done;
  switch (B) {
    case 1: return run_lmhead_b<1>(p, ids, max_logit, stream);
    case 2: return run_lmhead_b<2>(p, ids, max_logit, stream);
    case 3: return run_lmhead_b<3>(p, ids, max_logit, stream);
    case 4: return run_lmhead_b<4>(p, ids, max_logit, stream);
    case 5: return run_lmhead_b<5>(p, ids, max_logit, stream);
    case 6: return run_lmhead_b<6>(p, ids, max_logit, stream);
    case 7: return run_lmhead_b<7>(p, ids, max_logit, stream);
    case 8: return run_lmhead_b<8>(p, ids, max_logit, stream);
    default: return hipErrorInvalidValue;
  }
}

namespace {

size_t q8_lds(int k, int B) { return (size_t)B * (k + k / kGroup) * 4; }

template <int S, int B, bool ARGMAX>
hipError_t launch_q8(GemvParams p, hipStream_t stream) {
  const int G = p.k / kGroup;
  p.lshift = log2_floor(G < kWave ? G : kWave);
  const size_t lds = q8_lds(p.k, B);
  static int resident = -1;  // per instantiation
  if (resident < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, q8_gemv_kernel<S, B, ARGMAX>, 256, lds) != hipSuccess ||
        n < 1)
      n = 1;
    resident = n;
  }
  const int64_t rows_per_wave_iter = (int64_t)(kWave >> p.lshift) * S;
  const int64_t iters = (p.rows + rows_per_wave_iter - 1) / rows_per_wave_iter;
  int64_t blocks = (iters + 3) / 4;
  int64_t max_blocks = (int64_t)device_cu_count() * resident;
  if (max_blocks > kMaxGemvBlocks) max_blocks = kMaxGemvBlocks;  // one resident round at most
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((q8_gemv_kernel<S, B, ARGMAX>), dim3((unsigned)blocks), dim3(256), lds, stream, p);
  return hipGetLastError();
}

// B = 1: the 8-bit GEMV with fused argmax; B = 2..8: the LM-head MFMA kernel on 8-bit codes.
template <int B>
hipError_t run_lmhead_q8_b(GemvParams& p, int32_t* ids, float* max_logit, hipStream_t stream) {
  p.ids = ids;
  p.max_logit = max_logit;
  if constexpr (B >= 2) {
    const size_t lds = gemv_lds(p.k, B);
    const int64_t wave_steps = (p.rows + 15) / 16;  // 16 rows per wave step; one resident round
    int64_t blocks = (wave_steps + 3) / 4;
    int64_t max_blocks = (int64_t)device_cu_count() * lmhead_mfma_resident<B, true>(lds);
    if (max_blocks > kMaxGemvBlocks) max_blocks = kMaxGemvBlocks;  // one resident round at most
    if (blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL((lmhead_mfma_q8_kernel<B>), dim3((int)blocks), dim3(256), lds, stream, p);
    return hipGetLastError();
  }
  return launch_q8<B <= 2 ? 2 : 1, B, true>(p, stream);
}

}  // namespace

size_t q8_gemv_lds_bytes(int k, int B) { return q8_lds(k, B); }

hipError_t run_q8_gemv(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
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
  return launch_q8<2, 1, false>(p, stream);
}

hipError_t run_lmhead_argmax_q8(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                                int64_t rows, int k, const uint16_t* X, int B, int32_t* ids, float* max_logit,
                                unsigned long long* keys, unsigned* done, hipStream_t stream) {
  GemvParams p{};
  p.codes = reinterpret_cast<const uint4*>(codes);
  p.scales = scales;
  p.biases = biases;
  p.rows = rows;
  p.k = k;
  p.x = X;
  p.keys = keys;
  p.done = done;
  switch (B) {
    case 1: return run_lmhead_q8_b<1>(p, ids, max_logit, stream);
    case 2: return run_lmhead_q8_b<2>(p, ids, max_logit, stream);
    case 3: return run_lmhead_q8_b<3>(p, ids, max_logit, stream);
    case 4: return run_lmhead_q8_b<4>(p, ids, max_logit, stream);
    case 5: return run_lmhead_q8_b<5>(p, ids, max_logit, stream);
    case 6: return run_lmhead_q8_b<6>(p, ids, max_logit, stream);
    case 7: return run_lmhead_q8_b<7>(p, ids, max_logit, stream);
    case 8: return run_lmhead_q8_b<8>(p, ids, max_logit, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4moe
