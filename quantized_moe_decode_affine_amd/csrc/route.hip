// Router (logits, softmax top-k, renormalised weights) for a block of tokens,
// and the stable counting sort that groups (token, slot) rows by expert for
// the prefill expert GEMM (lily-qwen3.8-flash-next README, "How the speed was
// achieved": prefill runs the expert GEMM over token-to-expert groups).
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "preprows.h"
#include "topk.h"

namespace q4moe {

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// logits[t][e] = X[t] . router[e]: bf16 MFMA 32x32x16, fp32 accumulation.
// Workgroup = 32 tokens x 64 experts, 8 waves: wave w computes the 32x32 block of
// expert half (w & 1) over K quarter (w >> 1); the quarters are summed through LDS in
// a fixed order.  Each 64-column K step of both operands goes through LDS: one
// 16-byte-per-lane load instruction reads 8 whole 128-byte row pieces (8 cache lines;
// a row per lane would touch 32 lines per instruction), and three steps are in flight.
// Inside a row the eight 16-byte pieces are XOR-rotated by row bits 1-3, so that the
// MFMA operand reads (a row per lane) spread over all banks.
constexpr int kRouterStages = 3;
constexpr int kRouterQuarterBytes = (32 + 64) * 128;  // one quarter's token and expert rows of a step
constexpr int kRouterOps = 6;                         // load instructions per wave and step

__device__ __forceinline__ int router_swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(512) void router_logits_kernel(const uint16_t* __restrict__ router,
                                                            const uint16_t* __restrict__ X, int64_t T, int E,
                                                            int H, float* __restrict__ logits) {
  // one array per stage, so that the compiler can tell a stage's reads from the loads
  // still filling another
  __shared__ __align__(16) uint8_t s_st0[4 * kRouterQuarterBytes], s_st1[4 * kRouterQuarterBytes],
      s_st2[4 * kRouterQuarterBytes];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int eh = wave & 1, kq = wave >> 1;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int eb = blockIdx.y * 64;
  const int steps = H >> 6;
  const int per_q = (steps + 3) >> 2;  // steps per quarter: every wave runs the same count
  const int q_first = kq * per_q;

  // This wave's share of each step's loads: token rows (2 x 8) and expert rows (4 x 8)
  // of its quarter; lane l takes row base + l/8, piece (l%8) ^ swz(row).
  const uint16_t* src[kRouterOps];
  int dst[kRouterOps];
#pragma unroll
  for (int j = 0; j < kRouterOps; ++j) {
    const bool tok = j < 2;
    const int blk = tok ? eh * 2 + j : eh * 4 + (j - 2);
    const int r = blk * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ router_swz(r);
    src[j] = tok ? X + min<int64_t>(t0 + r, T - 1) * H + piece * 8
                 : router + (int64_t)min(eb + r, E - 1) * H + piece * 8;
    dst[j] = kq * kRouterQuarterBytes + (tok ? 0 : 32 * 128) + blk * 1024;
  }
  auto stage = [&](int st) -> uint8_t* { return st == 0 ? s_st0 : st == 1 ? s_st1 : s_st2; };
  // Steps past the quarter's end load the quarter's (or the matrix's) last step again
  // and are not computed: every wave issues the same loads per iteration.
  auto issue = [&](int i, int st) {
    const int s = min(q_first + min(i, per_q - 1), steps - 1);
#pragma unroll
    for (int j = 0; j < kRouterOps; ++j)
      __builtin_amdgcn_global_load_lds(src[j] + s * 64, stage(st) + dst[j], 16, 0, 0);
  };

  const int m = lane & 31, h = lane >> 5;
  const int a_row = m, b_row = 32 + eh * 32 + m;  // rows inside the quarter's region
  f32x16_t acc = {};
  // kGuard: some quarter has fewer steps than the others (H / 64 not a multiple of 4),
  // so a wave checks each step before computing it
  auto step = [&](int i, auto st_c, auto guard_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    constexpr bool kGuard = decltype(guard_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(kRouterOps * (kRouterStages - 2)));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(i + kRouterStages - 1, (st + kRouterStages - 1) % kRouterStages);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* base = stage(st) + kq * kRouterQuarterBytes;
    uint4 av[4], bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 2 * q + h;  // the 8 columns 8c..8c+7 of the step
      av[q] = *reinterpret_cast<const uint4*>(base + a_row * 128 + ((c ^ router_swz(a_row)) << 4));
      bv[q] = *reinterpret_cast<const uint4*>(base + b_row * 128 + ((c ^ router_swz(b_row)) << 4));
    }
    // all eight reads go out before the first MFMA waits (left alone, the scheduler
    // pairs each MFMA with its two reads and waits four times)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      asm volatile("" : "+v"(av[q].x), "+v"(av[q].y), "+v"(av[q].z), "+v"(av[q].w), "+v"(bv[q].x), "+v"(bv[q].y),
                   "+v"(bv[q].z), "+v"(bv[q].w));
    if (!kGuard || q_first + i < steps) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[q]),
                                                      __builtin_bit_cast(bf16x8_t, bv[q]), acc, 0, 0, 0);
    }
  };
  auto run = [&](auto guard_c) __attribute__((always_inline)) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    int i = 0;
    for (; i + kRouterStages <= per_q; i += kRouterStages) {
      step(i, S0{}, guard_c);
      step(i + 1, S1{}, guard_c);
      step(i + 2, S2{}, guard_c);
    }
    if (i < per_q) step(i, S0{}, guard_c);
    if (i + 1 < per_q) step(i + 1, S1{}, guard_c);
  };
  issue(0, 0);
  issue(1, 1);
  if (4 * per_q == steps)
    run(std::false_type{});
  else
    run(std::true_type{});
  // the repeated loads of the last steps are still landing in the stages
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16_t* s_part = reinterpret_cast<f32x16_t*>(s_st0);  // [3][2][64], the stages are idle now
  if (kq > 0) s_part[((kq - 1) * 2 + eh) * kWave + lane] = acc;
  __syncthreads();
  if (kq > 0) return;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const f32x16_t o = s_part[(j * 2 + eh) * kWave + lane];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] += o[k];
  }
  // D layout: column (expert) = lane % 32, row (token) = 8*(i/4) + 4*(lane/32) + i%4
  const int e = eb + eh * 32 + m;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t t = t0 + 8 * (k >> 2) + 4 * h + (k & 3);
    if (t < T && e < E) logits[t * E + e] = acc[k];
  }
}

template <int V>
__global__ __launch_bounds__(256) void topk_rows_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ int32_t s_ids[4][kMaxTopK];
  __shared__ float s_w[4][kMaxTopK];
  const int wave = threadIdx.x / kWave;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  wave_topk_sorted<V>(logits + t * E, E, k, s_ids[wave], s_w[wave]);
  const int lane = lane_id();
  if (lane < k) {
    ids[t * k + lane] = s_ids[wave][lane];
    weights[t * k + lane] = s_w[wave][lane];
  }
}

// ---- stable counting sort by expert, in two launches
// chunk_rank_kernel: workgroup c takes rows [c*kRankChunk, (c+1)*kRankChunk) in
// order and gives each row its rank among the chunk's earlier rows of the same
// expert; it writes the chunk's histogram hist[c][e].
// expert_scatter_kernel: workgroup c adds the counts of expert e in chunks
// before c (so a row's rank counts every earlier row of its expert: the order
// inside a segment is increasing r, stable and independent of scheduling), scans
// the per-expert totals into segment offsets (workgroup 0 also writes them out)
// and places its chunk's rows.

constexpr int kRankThreads = 256;
constexpr int kRankChunk = kMaxExperts;  // rows per chunk: one per thread of the scatter kernel

// Workgroups from nchunks on prepare rows (PrepRowsJob) instead: work of their own that
// only shares the launch, so that it runs beside the few rank workgroups.
__global__ __launch_bounds__(kRankThreads) void chunk_rank_kernel(const int32_t* __restrict__ ids, int64_t rows, int E,
                                                                  int32_t* __restrict__ local_rank,
                                                                  int32_t* __restrict__ hist, int nchunks,
                                                                  PrepRowsJob prep) {
  __shared__ int32_t s_cnt[kMaxExperts];
  if ((int)blockIdx.x >= nchunks) {
    prep::prep_rows_body<uint16_t>(prep.A, prep.rows, prep.K, prep.Gp, prep.out, prep.sums, prep.exps,
                                   prep::SplitRows{nullptr, INT64_MAX, 0, 1}, (int64_t)blockIdx.x - nchunks,
                                   (int64_t)gridDim.x - nchunks);
    return;
  }
  for (int e = threadIdx.x; e < E; e += kRankThreads) s_cnt[e] = 0;
  __syncthreads();
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const uint64_t below = (1ull << lane) - 1ull;  // lanes before this one
  const int64_t c0 = (int64_t)blockIdx.x * kRankChunk;
  constexpr int kSubs = kRankChunk / kRankThreads;
  int ids_sub[kSubs];  // this thread's rows' experts, all loaded before the first barrier
#pragma unroll
  for (int sub = 0; sub < kSubs; ++sub) {
    const int64_t r = c0 + sub * kRankThreads + threadIdx.x;
    ids_sub[sub] = ids[min(r, rows - 1)];
  }
#pragma unroll
  for (int sub = 0; sub < kSubs; ++sub) {  // 256 rows at a time, in row order
    const int64_t r = c0 + sub * kRankThreads + threadIdx.x;
    const int e = r < rows ? ids_sub[sub] : -1;
    const bool valid = e >= 0 && e < E;
    const uint32_t key = valid ? (uint32_t)e : 1024u;  // E <= 1024: 11 key bits
    uint64_t same = ~0ull;  // lanes of this wave holding the same key
#pragma unroll
    for (int bit = 0; bit < 11; ++bit) {
      const uint64_t ones = __ballot((key >> bit) & 1u);
      same &= ((key >> bit) & 1u) ? ones : ~ones;
    }
    const int before_in_wave = __popcll(same & below);
    const bool leader = (same & below) == 0;  // first lane of its key in this wave
    for (int w = 0; w < kRankThreads / kWave; ++w) {  // the waves' rows are in order: wave 0 first
      if (wave == w && valid) {
        const int32_t base = s_cnt[e];
        if (r < rows) local_rank[r] = base + before_in_wave;
        // every lane of the group has read base before the group leader moves it on
        __builtin_amdgcn_wave_barrier();
        if (leader) s_cnt[e] = base + __popcll(same);
      }
      __syncthreads();
    }
  }
  for (int e = threadIdx.x; e < E; e += kRankThreads) hist[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

__global__ __launch_bounds__(1024) void expert_scatter_kernel(const int32_t* __restrict__ ids, int64_t rows, int E,
                                                              const int32_t* __restrict__ local_rank,
                                                              const int32_t* __restrict__ hist, int nchunks,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_rows,
                                                              int32_t* __restrict__ inv_rows, GroupTiles tiles) {
  __shared__ int32_t s_c[kMaxExperts];
  __shared__ int32_t s_t[kMaxExperts];
  __shared__ int32_t s_before[kMaxExperts];  // rows of expert i in chunks before this workgroup's
  const int i = threadIdx.x;  // blockDim.x == kMaxExperts == kRankChunk
  const bool tiled = tiles.table != nullptr;
  const int tr = tiled ? tiles.tile_rows : 1;
  int32_t c = 0, before = 0;
  if (i < E)
    for (int ch0 = 0; ch0 < nchunks; ch0 += 16) {  // 16 chunks' counts in flight at once
      int32_t h[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) h[j] = hist[(int64_t)min(ch0 + j, nchunks - 1) * E + i];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int ch = ch0 + j;
        if (ch < nchunks) {
          before += ch < (int)blockIdx.x ? h[j] : 0;
          c += h[j];
        }
      }
    }
  s_before[i] = before;
  s_c[i] = c;
  s_t[i] = (c + tr - 1) / tr;
  __syncthreads();
  for (int off = 1; off < kMaxExperts; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t a = i >= off ? s_c[i - off] : 0;
    const int32_t b = i >= off ? s_t[i - off] : 0;
    __syncthreads();
    s_c[i] += a;
    s_t[i] += b;
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    if (i < E) offsets[i + 1] = s_c[i];
    if (i == 0) offsets[0] = 0;
    if (tiled) {
      // routed tiles of expert i, then the extra tiles, then unused slots
      if (i < E) {
        const int32_t t0 = i > 0 ? s_t[i - 1] : 0, p0 = i > 0 ? s_c[i - 1] : 0;
        for (int32_t t = t0; t < s_t[i]; ++t) {
          const int32_t first = p0 + (t - t0) * tr;
          tiles.table[t] = make_int4(i, first, min(tr, s_c[i] - first), 0);
        }
      }
      const int32_t routed = s_t[E - 1];
      for (int32_t t = routed + i; t < tiles.max_tiles; t += blockDim.x) {
        const int64_t first = (int64_t)(t - routed) * tr;
        tiles.table[t] = first < tiles.extra_rows
                             ? make_int4(-1, (int32_t)(rows + first), (int32_t)min<int64_t>(tr, tiles.extra_rows - first), 0)
                             : make_int4(-2, 0, 0, 0);
      }
    }
  }
  {
    const int64_t r = (int64_t)blockIdx.x * kRankChunk + threadIdx.x;  // this workgroup's chunk, one row per thread
    const int e = r < rows ? ids[r] : -1;
    if (e < 0 || e >= E) return;
    const int32_t pos = (e > 0 ? s_c[e - 1] : 0) + s_before[e] + local_rank[r];
    sorted_rows[pos] = (int32_t)r;
    inv_rows[r] = pos;
    if (tiled) {
      tiles.row_src[pos] = (int32_t)(r / tiles.topk);
      tiles.row_w[pos] = tiles.weights ? tiles.weights[r] : 1.0f;
    }
  }
}

int grid_for(int64_t n, int block) {
  int64_t b = (n + block - 1) / block;
  if (b > 65536) b = 65536;
  return (int)(b < 1 ? 1 : b);
}

// Router logits from an 8-bit affine router on bf16 matrix cores: the tiling of
// router_logits_kernel (32 tokens x 64 experts, 8 waves = 2 expert halves x 4 K
// quarters, operands of each step staged through LDS), whose 64-column K steps are
// exactly the quantization groups.  Codes 0..255 are exact in bfloat16 (the high half
// of their fp32 value), so each group's sum(x q) comes exact-product, fp32-summed from
// 4 MFMAs into a fresh accumulator; 4 more against all-ones codes give the group's
// token sums sum(x) in the same layout, and the group is folded as
// acc += scale * sum(x q) + bias * sum(x).  A code row's 64 bytes of a group are four
// 16-byte pieces, XOR-rotated by row bits 2-3.
__device__ __forceinline__ bf16x8_t bytes_to_bf16x8(uint2 c) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = i < 2 ? c.x : c.y;
    const int sh = 16 * (i & 1);
    const uint32_t lo = __float_as_uint((float)((w >> sh) & 0xFFu)) >> 16;
    const uint32_t hi = __float_as_uint((float)((w >> (sh + 8)) & 0xFFu)) & 0xFFFF0000u;
    o[i] = lo | hi;
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

constexpr int kQ8RouterQuarterBytes = 32 * 128;  // a quarter's token rows (128 B each) of a step; its code rows
                                                 // (64 B each) sit in arrays of their own
constexpr int kQ8RouterOps = 6;  // per wave and step: 2 token-row and 2 code-row loads, the scale and the bias

__device__ __forceinline__ int code_swz(int r) { return (r >> 2) & 3; }

__global__ __launch_bounds__(512) void q8_router_logits_kernel(Q4Mat R, const uint16_t* __restrict__ X, int64_t T,
                                                               int E, int H, float* __restrict__ logits) {
  __shared__ __align__(16) uint8_t s_st0[4 * kQ8RouterQuarterBytes], s_st1[4 * kQ8RouterQuarterBytes],
      s_st2[4 * kQ8RouterQuarterBytes];
  __shared__ __align__(16) uint8_t s_cd0[4 * 64 * 64], s_cd1[4 * 64 * 64], s_cd2[4 * 64 * 64];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int eh = wave & 1, kq = wave >> 1;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int eb = blockIdx.y * 64;
  const int G = H >> 6;
  const int per_q = (G + 3) >> 2;
  const int q_first = kq * per_q;
  const int m = lane & 31, h = lane >> 5;
  const int erow = min(eb + eh * 32 + m, E - 1);  // this lane's expert (its output column)

  // loads of this wave: token rows (eh*2 + j)*8 + lane/8, piece (lane%8)^swz; code rows
  // (eh*2 + j)*16 + lane/4, piece (lane%4)^swz
  const uint16_t* xsrc[2];
  const uint8_t* csrc[2];
  int xdst[2], cdst[2];
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(R.codes);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int xb = eh * 2 + j, xr = xb * 8 + (lane >> 3);
    xsrc[j] = X + min<int64_t>(t0 + xr, T - 1) * H + ((lane & 7) ^ router_swz(xr)) * 8;
    xdst[j] = kq * kQ8RouterQuarterBytes + xb * 1024;
    const int cb = eh * 2 + j, cr = cb * 16 + (lane >> 2);
    csrc[j] = codes + (int64_t)min(eb + cr, E - 1) * H + ((lane & 3) ^ code_swz(cr)) * 16;
    cdst[j] = kq * 64 * 64 + cb * 1024;
  }
  const uint16_t* sc = R.scales + (int64_t)erow * G;
  const uint16_t* bi = R.biases + (int64_t)erow * G;
  auto stage = [&](int st) -> uint8_t* { return st == 0 ? s_st0 : st == 1 ? s_st1 : s_st2; };
  auto cstage = [&](int st) -> uint8_t* { return st == 0 ? s_cd0 : st == 1 ? s_cd1 : s_cd2; };
  uint32_t scv[kRouterStages], biv[kRouterStages];  // raw bf16 scale and bias of the group in each stage
  // ga: the step's load addresses, returned so that the caller can keep them live past
  // its LDS reads (the compiler waits for every load in flight before it reuses a load's
  // address registers, e.g. as an LDS read's destination)
  auto issue = [&](int i, int st, uintptr_t (&ga)[6]) {
    const int g = min(q_first + min(i, per_q - 1), G - 1);
    ga[4] = reinterpret_cast<uintptr_t>(sc + g);
    ga[5] = reinterpret_cast<uintptr_t>(bi + g);
    scv[st] = *reinterpret_cast<const uint16_t*>(ga[4]);
    biv[st] = *reinterpret_cast<const uint16_t*>(ga[5]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ga[2 * j] = reinterpret_cast<uintptr_t>(xsrc[j] + g * 64);
      ga[2 * j + 1] = reinterpret_cast<uintptr_t>(csrc[j] + g * 64);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ga[2 * j]), stage(st) + xdst[j], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ga[2 * j + 1]), cstage(st) + cdst[j], 16, 0, 0);
    }
  };

  const int a_row = m, b_row = eh * 32 + m;
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 1.0 pairs
  f32x16_t acc = {};
  auto step = [&](int i, auto st_c, auto guard_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    constexpr bool kGuard = decltype(guard_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(kQ8RouterOps * (kRouterStages - 2)));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uintptr_t ga[6];
    issue(i + kRouterStages - 1, (st + kRouterStages - 1) % kRouterStages, ga);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* xb = stage(st) + kq * kQ8RouterQuarterBytes;
    const uint8_t* cbp = cstage(st) + kq * 64 * 64;
    uint4 av[4];
    uint2 bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 2 * q + h;  // columns 8c..8c+7 of the group
      av[q] = *reinterpret_cast<const uint4*>(xb + a_row * 128 + ((c ^ router_swz(a_row)) << 4));
      const uint4 cw = *reinterpret_cast<const uint4*>(cbp + b_row * 64 + ((q ^ code_swz(b_row)) << 4));
      bv[q] = h ? make_uint2(cw.z, cw.w) : make_uint2(cw.x, cw.y);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      asm volatile("" : "+v"(av[q].x), "+v"(av[q].y), "+v"(av[q].z), "+v"(av[q].w), "+v"(bv[q].x), "+v"(bv[q].y));
#pragma unroll
    for (int j = 0; j < 6; ++j) asm volatile("" ::"v"(ga[j]));
    if (!kGuard || q_first + i < G) {
      f32x16_t pq = {}, px = {};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[q]), bytes_to_bf16x8(bv[q]), pq,
                                                     0, 0, 0);
        px = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[q]),
                                                     __builtin_bit_cast(bf16x8_t, ones), px, 0, 0, 0);
      }
      const float s = bf16_bits_to_f32(scv[st]), o = bf16_bits_to_f32(biv[st]);
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] += fmaf(s, pq[k], o * px[k]);
    }
  };
  auto run = [&](auto guard_c) __attribute__((always_inline)) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    int i = 0;
    for (; i + kRouterStages <= per_q; i += kRouterStages) {
      step(i, S0{}, guard_c);
      step(i + 1, S1{}, guard_c);
      step(i + 2, S2{}, guard_c);
    }
    if (i < per_q) step(i, S0{}, guard_c);
    if (i + 1 < per_q) step(i + 1, S1{}, guard_c);
  };
  {
    uintptr_t ga[6];
    issue(0, 0, ga);
    issue(1, 1, ga);
  }
  if (4 * per_q == G)
    run(std::false_type{});
  else
    run(std::true_type{});
  __builtin_amdgcn_s_waitcnt(0);  // the repeated loads of the last steps are still landing
  __syncthreads();

  // quarters 1..3 hand their sums to quarter 0 through the idle stages ([2][64] each:
  // quarters 1 and 2 in stage 0, quarter 3 in stage 1)
  auto s_part = [&](int j) -> f32x16_t* {
    return j < 2 ? reinterpret_cast<f32x16_t*>(s_st0) + j * 2 * kWave : reinterpret_cast<f32x16_t*>(s_st1);
  };
  static_assert(4 * kQ8RouterQuarterBytes >= 2 * 2 * kWave * 64, "two quarters' sums fit a stage");
  if (kq > 0) s_part(kq - 1)[eh * kWave + lane] = acc;
  __syncthreads();
  if (kq > 0) return;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const f32x16_t o = s_part(j)[eh * kWave + lane];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] += o[k];
  }
  // D layout: column (expert) = lane % 32, row (token) = 8*(i/4) + 4*(lane/32) + i%4
  const int e = eb + eh * 32 + m;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t t = t0 + 8 * (k >> 2) + 4 * h + (k & 3);
    if (t < T && e < E) logits[t * E + e] = acc[k];
  }
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int n_experts) { return align256((size_t)T * n_experts * 4); }

hipError_t run_route_topk(const uint16_t* router, int E, int H, const uint16_t* X, int64_t T, int k, int32_t* ids,
                          float* weights, void* ws, hipStream_t stream, const Q4Mat* router_q8) {
  float* logits = static_cast<float*>(ws);
  dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 63) / 64));
  if (router_q8 && router_q8->codes)
    hipLaunchKernelGGL(q8_router_logits_kernel, grid, dim3(512), 0, stream, *router_q8, X, T,
                       E, H, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(512), 0, stream, router, X, T, E, H, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 tgrid((unsigned)((T + 3) / 4)), tthreads(256);
  if (E <= 4 * kWave)
    hipLaunchKernelGGL(topk_rows_kernel<4>, tgrid, tthreads, 0, stream, logits, T, E, k, ids, weights);
  else if (E <= 8 * kWave)
    hipLaunchKernelGGL(topk_rows_kernel<8>, tgrid, tthreads, 0, stream, logits, T, E, k, ids, weights);
  else
    hipLaunchKernelGGL(topk_rows_kernel<kMaxExperts / kWave>, tgrid, tthreads, 0, stream, logits, T, E, k, ids,
                       weights);
  return hipGetLastError();
}

size_t permute_workspace_bytes(int64_t rows, int n_experts) {
  const int64_t nchunks = (rows + kRankChunk - 1) / kRankChunk;
  return align256((size_t)rows * 4) + align256((size_t)(nchunks > 0 ? nchunks : 1) * n_experts * 4);
}

int group_max_tiles(int64_t rows, int n_experts, int64_t extra_rows, int tile_rows) {
  return (int)((rows + tile_rows - 1) / tile_rows + n_experts + (extra_rows + tile_rows - 1) / tile_rows);
}

hipError_t run_permute(const int32_t* ids, int64_t rows, int E, int32_t* offsets, int32_t* sorted_rows,
                       int32_t* inv_rows, void* ws, const GroupTiles* tiles, hipStream_t stream,
                       const PrepRowsJob* prep) {
  char* w = static_cast<char*>(ws);
  const int nchunks = (int)((rows + kRankChunk - 1) / kRankChunk);
  int32_t* local_rank = reinterpret_cast<int32_t*>(w);
  int32_t* hist = reinterpret_cast<int32_t*>(w + align256((size_t)rows * 4));
  GroupTiles none{};
  // the row preparation's workgroups (one wave per row) after the rank workgroups
  const PrepRowsJob pj = prep ? *prep : PrepRowsJob{};
  const int64_t prep_blocks = prep && prep->rows > 0 ? std::min<int64_t>((prep->rows + 3) / 4, 8192) : 0;
  if (nchunks == 0) {  // no rows: offsets and the tile table still get written
    if (prep_blocks > 0) {
      hipLaunchKernelGGL(chunk_rank_kernel, dim3((unsigned)prep_blocks), dim3(kRankThreads), 0, stream, ids, rows, E,
                         local_rank, hist, 0, pj);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(expert_scatter_kernel, dim3(1), dim3(kMaxExperts), 0, stream, ids, rows, E, local_rank, hist,
                       0, offsets, sorted_rows, inv_rows, tiles ? *tiles : none);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(chunk_rank_kernel, dim3((unsigned)(nchunks + prep_blocks)), dim3(kRankThreads), 0, stream, ids,
                     rows, E, local_rank, hist, nchunks, pj);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(expert_scatter_kernel, dim3(nchunks), dim3(kMaxExperts), 0, stream, ids, rows, E, local_rank,
                     hist, nchunks, offsets, sorted_rows, inv_rows, tiles ? *tiles : none);
  return hipGetLastError();
}

}  // namespace q4moe
