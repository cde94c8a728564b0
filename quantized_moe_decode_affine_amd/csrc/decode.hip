// Batch-1 decode step of one MoE feed-forward layer in one launch.
//
// The step is a dependent chain of weight streams (lily-qwen3.8-flash-next
// README, "How the speed was achieved": decode is bandwidth-bound and its
// kernels are tuned against the chain of reads).  One grid of one workgroup
// per CU runs three phases:
//   A: router logits (bf16 GEMV, one row per wave 0 of a workgroup), each
//      published with this launch's epoch in one 64-bit word, while waves 1-3
//      compute the shared expert's gate/up rows with SwiGLU (off the critical
//      path: their results are needed only in phase C);
//   B: top-k of the logits (recomputed by every workgroup straight from the
//      tagged words, so seeing a logit and reading it are one load), then the
//      routed experts' gate/up rows with SwiGLU; meanwhile each workgroup
//      prefetches into registers the down-projection weights of the output
//      rows it owns in phase C (known once the experts are);
//   C: for each owned output row, the down rows of all selected experts and
//      the shared expert, split over the workgroup's waves, combined in LDS in
//      a fixed order (no atomics); y is written once.
//
// No grid-wide barrier.  The logits carry the epoch themselves.  For the SwiGLU
// activations each workgroup, when its phase A/B work is done and its
// device-coherent stores have landed, publishes one flag word (the epoch); a
// consumer polls the 256-ish flags, then reads the activations once with
// device-coherent loads.  The epoch is agreed through
// per-group arrival counters in the workspace.  Every poll is bounded: a lost
// flag yields a wrong result and a recorded timeout, never a hang.
#include "kernels.h"
#include "topk.h"
#include "vecstage.h"

namespace q4moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kEpochGroups = 8;
constexpr int kPrefetchSlots = 3;   // down-row prefetch: slots per wave held in registers
constexpr int kStageRounds = 3;     // phase C staging: 8-value blocks per thread with loads in flight (9 x 512 values in one pass)
constexpr unsigned kPollLimit = 1u << 18;  // ~0.25 s of polling

constexpr int kMaxBlocks = 1024;
constexpr int kFlagStride = 16;  // 64 bytes

struct DecodeWs {
  unsigned long long group_ctr[kEpochGroups][32];  // {epoch:hi32, arrivals:lo32}, one 256-byte slot each
  unsigned timeouts;
  unsigned pad[63];
  // Router logit of expert e: tag_logit[e][0] = {epoch:hi32, fp32 bits:lo32}.
  // One 64-byte line per word (and per flag below): words that share a line
  // are written by different CUs, and such partial-line stores slow their
  // observers down severalfold.
  unsigned long long tag_logit[kMaxExperts][8];
  // flag_b[b][0] is the epoch once workgroup b's activations are visible.
  unsigned flag_b[kMaxBlocks][kFlagStride];
};

struct DecodeParams {
  DecodeLayer L;
  const uint16_t* x;          // [H]
  void* y;                    // [H]
  int out_bf16;
  int32_t* ids_out;           // nullable [k]
  float* w_out;               // nullable [k]
  DecodeWs* ws;
  float* act;                 // [k+1][I]: routed slots 0..k-1, shared slot k
  int lsH;                    // log2 lanes per row for rows of length hidden
  int lsI;                    // log2 lanes per row for rows of length inter
};

// Publish this workgroup's phase flag once every thread's device-coherent stores
// have completed.
__device__ __forceinline__ void publish_flag(unsigned* flag, uint32_t epoch) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave waits until flags[i][0] for i < n all equal `epoch` (bounded).
__device__ __forceinline__ void wave_wait_flags(const unsigned (*flag_rows)[kFlagStride], int n, uint32_t epoch,
                                                unsigned* timeouts) {
  const unsigned* flags = &flag_rows[0][0];
  const int lane = lane_id();
  for (unsigned spins = 0;; ++spins) {
    bool ready = true;
    for (int base = 0; base < n; base += 4 * kWave) {
      unsigned f[4];  // four loads in flight per lane (clamped index, results past n ignored)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        f[q] = __hip_atomic_load(const_cast<unsigned*>(flags + kFlagStride * min(base + q * kWave + lane, n - 1)), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int q = 0; q < 4; ++q) ready &= base + q * kWave + lane >= n || f[q] == epoch;
    }
    if (__all(ready)) break;
    if (spins == kPollLimit) {
      if (lane == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Stage a bf16 vector of n values (n % 32 == 0) into LDS: threads [t0, t0 + nthr)
// take one 8-value block each per pass, chunk sums by a quad reduction (nthr and
// t0 multiples of 4, so the 4 blocks of a chunk sit in one lane quad).
__device__ __forceinline__ void stage_bf16_parallel(const uint16_t* __restrict__ x, int n, uint32_t* vp, float* vs,
                                                    int t0, int nthr) {
  constexpr int ST = chunk_stride<1>();
  const int t = threadIdx.x - t0;
  if (t < 0 || t >= nthr) return;
  const int nblk = n >> 3;
  for (int base = 0; base < nblk; base += nthr) {
    const int b = base + t;
    float sum = 0.f;
    if (b < nblk) {
      const uint4 v = reinterpret_cast<const uint4*>(x)[b];
      sum = (bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16)) +
            (bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16)) +
            (bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16)) +
            (bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16));
      *reinterpret_cast<uint4*>(vp + (b >> 2) * ST + (b & 3) * 4) = permute_block(v);
    }
    sum = group_sum_rt(sum, 2);
    if (b < nblk && (b & 3) == 0) vs[b >> 2] = sum;
  }
}

// Convert 8 fp32 values into the hi/lo permuted pair layout of one 8-value block.
__device__ __forceinline__ float store_split_block(const float (&v)[8], uint32_t* dst) {
  uint32_t hi[8], lo[8];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    hi[j] = f32_to_bf16_bits(v[j]);
    const float h = bf16_bits_to_f32(hi[j]);
    lo[j] = f32_to_bf16_bits(v[j] - h);
    sum += h + bf16_bits_to_f32(lo[j]);
  }
  *reinterpret_cast<uint4*>(dst) =
      make_uint4(hi[0] | hi[4] << 16, hi[1] | hi[5] << 16, hi[2] | hi[6] << 16, hi[3] | hi[7] << 16);
  *reinterpret_cast<uint4*>(dst + 16) =
      make_uint4(lo[0] | lo[4] << 16, lo[1] | lo[5] << 16, lo[2] | lo[6] << 16, lo[3] | lo[7] << 16);
  return sum;
}

// Stage `nvec` fp32 vectors of n values each (contiguous, written by other
// workgroups) as hi/lo bf16 parts: threads [t0, t0 + nthr) take 8-value blocks,
// kStageRounds blocks per thread with all loads issued first.  nthr must be a
// multiple of 4 (the 4 blocks of a chunk sit in one lane quad).
__device__ __forceinline__ void stage_coherent_split(const float* src, int nvec, int n, uint32_t* vp, float* vs,
                                                     int t0, int nthr) {
  constexpr int ST = chunk_stride<2>();
  const int t = threadIdx.x - t0;
  if (t < 0 || t >= nthr) return;
  const int nblk = (nvec * n) >> 3;
  for (int base = 0; base < nblk; base += nthr * kStageRounds) {
    float v[kStageRounds][8];
#pragma unroll
    for (int r = 0; r < kStageRounds; ++r) {
      const int b = base + r * nthr + t;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[r][j] = ld_agent(src + 8 * min(b, nblk - 1) + j);
    }
#pragma unroll
    for (int r = 0; r < kStageRounds; ++r) {
      const int b = base + r * nthr + t;
      float sum = 0.f;
      if (b < nblk) sum = store_split_block(v[r], vp + (b >> 2) * ST + (b & 3) * 4);
      sum = group_sum_rt(sum, 2);
      if (b < nblk && (b & 3) == 0) vs[b >> 2] = sum;
    }
  }
}

// Gate/up row pointers of row i of expert e (e indexes the stacked matrices).
struct GateUpRef {
  const uint4* gc;
  const uint4* uc;
  const uint16_t *gs, *gb, *us, *ub;
};

__device__ __forceinline__ GateUpRef gate_up_ref(const Q4Mat& gm, const Q4Mat& um, int64_t e, int i, int H, int I) {
  const int C = H >> 5, G = H >> 6;
  const int64_t oc = e * (int64_t)I * (H >> 3), og = e * (int64_t)I * G;
  GateUpRef r;
  r.gc = reinterpret_cast<const uint4*>(gm.codes + oc) + (int64_t)i * C;
  r.uc = reinterpret_cast<const uint4*>(um.codes + oc) + (int64_t)i * C;
  r.gs = gm.scales + og + (int64_t)i * G;
  r.gb = gm.biases + og + (int64_t)i * G;
  r.us = um.scales + og + (int64_t)i * G;
  r.ub = um.biases + og + (int64_t)i * G;
  return r;
}

// NI independent (gate row, up row) items against the staged x, loads of all
// items issued before any arithmetic; every lane of a row's lane group returns (g, u).
template <int NI>
__device__ __forceinline__ void gate_up_dot(const GateUpRef (&ref)[NI], const bool (&live)[NI], int H, int sub,
                                            int L, int lsh, const uint32_t* vp, const float* vs, float2 (&out)[NI]) {
  constexpr int ST = chunk_stride<1>();
  const int G = H >> 6;
  float ag[NI], au[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) ag[n] = au[n] = 0.f;
  for (int g = sub; g < G; g += L) {
    uint4 g0[NI], g1[NI], u0[NI], u1[NI];
    uint32_t gsb[NI], gbb[NI], usb[NI], ubb[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      if (live[n]) {
        g0[n] = ref[n].gc[2 * g];
        g1[n] = ref[n].gc[2 * g + 1];
        u0[n] = ref[n].uc[2 * g];
        u1[n] = ref[n].uc[2 * g + 1];
        gsb[n] = ref[n].gs[g];
        gbb[n] = ref[n].gb[g];
        usb[n] = ref[n].us[g];
        ubb[n] = ref[n].ub[g];
      } else {
        g0[n] = g1[n] = u0[n] = u1[n] = make_uint4(0, 0, 0, 0);
        gsb[n] = gbb[n] = usb[n] = ubb[n] = 0;
      }
    }
    const uint32_t* v = vp + 2 * g * ST;
    const float vsum = vs[2 * g] + vs[2 * g + 1];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      ag[n] += affine_term(chunk_pdot<1>(g0[n], v) + chunk_pdot<1>(g1[n], v + ST), vsum, gsb[n], gbb[n]);
      au[n] += affine_term(chunk_pdot<1>(u0[n], v) + chunk_pdot<1>(u1[n], v + ST), vsum, usb[n], ubb[n]);
    }
  }
#pragma unroll
  for (int n = 0; n < NI; ++n) out[n] = make_float2(group_sum_rt(ag[n], lsh), group_sum_rt(au[n], lsh));
}

// Top-k of E logits by one wave, polling the epoch-tagged words that other
// workgroups publish until every one carries `epoch` (bounded; a timeout is
// counted).  Lane l holds ids [l*V, l*V + V) with its keys sorted in descending
// order, so each of the k rounds is a wave-wide maximum of the lane heads and a
// pop in the winning lane.  Equal logits resolve to the lower expert id: inside
// a lane by the sort order, across lanes because the lowest matching lane wins.
// Writes ids/weights (renormalised softmax of the kept logits) to LDS and, when
// given, to ids_out/w_out.
template <int V>
__device__ __forceinline__ void wave_topk_tagged(const unsigned long long (*tags)[8], int E, int k, uint32_t epoch,
                                                 unsigned* timeouts, int32_t* s_ids, float* s_w, int32_t* ids_out,
                                                 float* w_out) {
  const int lane = lane_id();
  uint32_t key[V];
  int id[V];
#pragma unroll
  for (int j = 0; j < V; ++j) id[j] = lane * V + j;
  for (unsigned spins = 0;; ++spins) {
    bool ready = true;
    unsigned long long t[V];
#pragma unroll
    for (int j = 0; j < V; ++j)  // all loads in flight together
      t[j] = __hip_atomic_load(const_cast<unsigned long long*>(&tags[min(id[j], E - 1)][0]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      key[j] = (uint32_t)t[j];
      ready &= id[j] >= E || (uint32_t)(t[j] >> 32) == epoch;
    }
    if (__all(ready)) break;
    if (spins == kPollLimit) {
      if (lane == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int j = 0; j < V; ++j) key[j] = id[j] < E ? float_key(__uint_as_float(key[j])) : 0u;
  // insertion sort, descending key; ties keep the lower id first (ids ascend with j)
#pragma unroll
  for (int a = 1; a < V; ++a)
#pragma unroll
    for (int b = a; b > 0; --b) {
      const bool sw = key[b] > key[b - 1];
      const uint32_t tk = key[b];
      const int ti = id[b];
      key[b] = sw ? key[b - 1] : key[b];
      id[b] = sw ? id[b - 1] : id[b];
      key[b - 1] = sw ? tk : key[b - 1];
      id[b - 1] = sw ? ti : id[b - 1];
    }
  float top = 0.f, my_val = 0.f;
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    const uint32_t m = wave_max_u32(key[0]);
    const int src = __builtin_ctzll(__ballot(key[0] == m));
    const int sel = __builtin_amdgcn_readlane(id[0], src);
    if (lane == src) {
#pragma unroll
      for (int j = 0; j + 1 < V; ++j) {
        key[j] = key[j + 1];
        id[j] = id[j + 1];
      }
      key[V - 1] = 0u;
    }
    const float v = key_float(m);
    if (r == 0) top = v;
    if (lane == r) {
      my_id = sel;
      my_val = v;
    }
  }
  const float ex = lane < k ? expf(my_val - top) : 0.f;
  const float sum = group_sum_rt(ex, 6);
  if (lane < k) {
    s_ids[lane] = my_id;
    s_w[lane] = ex / sum;
    if (ids_out) ids_out[lane] = my_id;
    if (w_out) w_out[lane] = ex / sum;
  }
}

struct DownPrefetch {
  uint4 c0, c1;
  uint32_t s, b;
};

__global__ __launch_bounds__(kThreads) void decode_layer_kernel(DecodeParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ int32_t s_ids[kMaxTopK + 1];
  __shared__ float s_w[kMaxTopK + 1];
  __shared__ float s_red[kWaves][kWave];
  __shared__ uint32_t s_epoch;

  const int H = p.L.hidden, I = p.L.inter, E = p.L.n_experts, k = p.L.top_k;
  const int CH = H >> 5, CI = I >> 5;
  const int nslot = k + (p.L.has_shared ? 1 : 0);
  uint32_t* xp = smem;                                                                // [CH][ST1]
  float* xs = reinterpret_cast<float*>(xp + CH * chunk_stride<1>());                   // [CH]
  uint32_t* ap = reinterpret_cast<uint32_t*>(xs + CH);                                // [nslot][CI][ST2]
  float* as = reinterpret_cast<float*>(ap + (size_t)nslot * CI * chunk_stride<2>());  // [nslot][CI]
  unsigned* timeouts = &p.ws->timeouts;

  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int gwave = blockIdx.x * kWaves + wv;
  const int nwaves = gridDim.x * kWaves;

  // ---- epoch of this launch: the arrivals of one group agree on its counter's
  // epoch field.  Taken by thread 0 once wave 0's first router loads are in
  // flight, so the two latencies overlap.
  uint32_t my_epoch = 0;
  auto acquire_epoch = [&]() {
    const int g = blockIdx.x % kEpochGroups;
    const unsigned gsize = (gridDim.x - g + kEpochGroups - 1) / kEpochGroups;
    unsigned long long* ctr = &p.ws->group_ctr[g][0];
    const unsigned long long old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)old == gsize - 1)
      __hip_atomic_fetch_add(ctr, (1ull << 32) - gsize, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    my_epoch = (uint32_t)(old >> 32) + 1u;
    s_epoch = my_epoch;
  };

  // ------------------------------------------------------------ phase A
  if (wv == 0) {
    // router rows e = blockIdx.x, blockIdx.x + gridDim.x, ...; x is read from global memory
    bool have_epoch = false;
    for (int it = blockIdx.x; it < E; it += gridDim.x) {
      const uint4* r = reinterpret_cast<const uint4*>(p.L.router + (size_t)it * H);
      const uint4* xv = reinterpret_cast<const uint4*>(p.x);
      constexpr int kBatch = 4;  // row chunks in flight per lane
      float acc0 = 0.f, acc1 = 0.f;
      for (int c0 = 0; c0 < (H >> 3); c0 += kBatch * kWave) {
        uint4 w[kBatch], v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const int c = c0 + q * kWave + lane;
          const bool ok = c < (H >> 3);
          w[q] = ok ? r[c] : make_uint4(0, 0, 0, 0);
          v[q] = ok ? xv[c] : make_uint4(0, 0, 0, 0);
        }
        if (!have_epoch) {
          have_epoch = true;
          if (lane == 0) acquire_epoch();
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          acc0 = dot2_bf16(w[q].x, v[q].x, acc0);
          acc1 = dot2_bf16(w[q].y, v[q].y, acc1);
          acc0 = dot2_bf16(w[q].z, v[q].z, acc0);
          acc1 = dot2_bf16(w[q].w, v[q].w, acc1);
        }
      }
      const float acc = group_sum_rt(acc0 + acc1, 6);
      const uint32_t ep = __builtin_amdgcn_readfirstlane(my_epoch);  // lane 0 holds it
      if (lane == 0)
        __hip_atomic_store(&p.ws->tag_logit[it][0], ((unsigned long long)ep << 32) | __float_as_uint(acc),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!have_epoch && lane == 0) acquire_epoch();
  } else {
    stage_bf16_parallel(p.x, H, xp, xs, kWave, kThreads - kWave);
  }
  __syncthreads();
  const uint32_t epoch = s_epoch;

  if (wv == 0) {
    // B: top-k from the tagged logits (every workgroup, redundantly)
    if (E <= 4 * kWave)
      wave_topk_tagged<4>(p.ws->tag_logit, E, k, epoch, timeouts, s_ids, s_w, blockIdx.x == 0 ? p.ids_out : nullptr,
                          blockIdx.x == 0 ? p.w_out : nullptr);
    else
      wave_topk_tagged<kMaxExperts / kWave>(p.ws->tag_logit, E, k, epoch, timeouts, s_ids, s_w,
                                            blockIdx.x == 0 ? p.ids_out : nullptr, blockIdx.x == 0 ? p.w_out : nullptr);
    if (lane == 0 && p.L.has_shared) {
      s_ids[k] = -1;
      s_w[k] = 1.0f;
    }
  } else if (p.L.has_shared) {
    // A, off the critical path: the shared expert's gate/up rows over waves 1-3 of every workgroup
    const int aw = (wv - 1) * gridDim.x + blockIdx.x, nw = (kWaves - 1) * gridDim.x;
    const int L = 1 << p.lsH, sub = lane & (L - 1), rsub = lane >> p.lsH, rpi = kWave >> p.lsH;
    const int pair_items = (I + rpi - 1) / rpi;
    for (int it = aw; it < pair_items; it += nw) {
      const int i = it * rpi + rsub;
      const bool live[1] = {i < I};
      const GateUpRef ref[1] = {gate_up_ref(p.L.sh_gate, p.L.sh_up, 0, live[0] ? i : 0, H, I)};
      float2 gu[1];
      gate_up_dot<1>(ref, live, H, sub, L, p.lsH, xp, xs, gu);
      if (live[0] && sub == 0) st_agent(p.act + (size_t)k * I + i, silu(gu[0].x) * gu[0].y);
    }
  }
  __syncthreads();

  // prefetch the down rows this workgroup owns in phase C (its first row block)
  const int LI = 1 << p.lsI, subI = lane & (LI - 1), rsubI = lane >> p.lsI, rpiI = kWave >> p.lsI;
  const int GI = I >> 6;
  const bool pf_ok = GI == LI && (int)blockIdx.x * rpiI < H;
  DownPrefetch pf[kPrefetchSlots];
  {
    const int n = blockIdx.x * rpiI + rsubI;
    const int64_t mat_codes = (int64_t)H * (I >> 3), mat_groups = (int64_t)H * GI;
#pragma unroll
    for (int s = 0; s < kPrefetchSlots; ++s) {
      const int j = wv + kWaves * s;
      if (pf_ok && j < nslot && n < H) {
        const int e = s_ids[j];
        const Q4Mat& m = e >= 0 ? p.L.down : p.L.sh_down;
        const int64_t oc = e >= 0 ? e * mat_codes : 0, og = e >= 0 ? e * mat_groups : 0;
        const uint4* cr = reinterpret_cast<const uint4*>(m.codes + oc) + (int64_t)n * CI;
        pf[s].c0 = cr[2 * subI];
        pf[s].c1 = cr[2 * subI + 1];
        pf[s].s = m.scales[og + (int64_t)n * GI + subI];
        pf[s].b = m.biases[og + (int64_t)n * GI + subI];
      } else {
        pf[s].c0 = pf[s].c1 = make_uint4(0, 0, 0, 0);
        pf[s].s = pf[s].b = 0;
      }
    }
  }

  {
    const int L = 1 << p.lsH, sub = lane & (L - 1), rsub = lane >> p.lsH, rpi = kWave >> p.lsH;
    const int per_slot = (I + rpi - 1) / rpi;
    const int items = k * per_slot;
    for (int it = gwave; it < items; it += 2 * nwaves) {
      int i[2], j[2];
      bool live[2];
      GateUpRef ref[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int t = it + n * nwaves;
        j[n] = t / per_slot;
        i[n] = (t - j[n] * per_slot) * rpi + rsub;
        live[n] = t < items && i[n] < I;
        ref[n] = gate_up_ref(p.L.gate, p.L.up, live[n] ? s_ids[j[n]] : 0, live[n] ? i[n] : 0, H, I);
      }
      float2 gu[2];
      gate_up_dot<2>(ref, live, H, sub, L, p.lsH, xp, xs, gu);
#pragma unroll
      for (int n = 0; n < 2; ++n)
        if (live[n] && sub == 0) st_agent(p.act + (size_t)j[n] * I + i[n], silu(gu[n].x) * gu[n].y);
    }
  }
  publish_flag(&p.ws->flag_b[blockIdx.x][0], epoch);

  // ------------------------------------------------------------ phase C
  if (wv == 0) wave_wait_flags(p.ws->flag_b, gridDim.x, epoch, timeouts);
  __syncthreads();
  stage_coherent_split(p.act, nslot, I, ap, as, 0, kThreads);  // routed slots and the shared slot
  __syncthreads();
  {
    constexpr int ST = chunk_stride<2>();
    const int64_t mat_codes = (int64_t)H * (I >> 3), mat_groups = (int64_t)H * GI;
    for (int rb = blockIdx.x; rb * rpiI < H; rb += gridDim.x) {
      const int n = rb * rpiI + rsubI;
      const bool first = rb == (int)blockIdx.x && pf_ok;
      float acc = 0.f;
      if (n < H) {
        for (int j = wv, s = 0; j < nslot; j += kWaves, ++s) {
          const int e = s_ids[j];
          float part = 0.f;
          if (first && s < kPrefetchSlots) {
            DownPrefetch d = pf[0];
#pragma unroll
            for (int q = 1; q < kPrefetchSlots; ++q)
              if (q == s) d = pf[q];
            const uint32_t* v = ap + ((size_t)j * CI + 2 * subI) * ST;
            const float vsum = as[j * CI + 2 * subI] + as[j * CI + 2 * subI + 1];
            part = affine_term(chunk_pdot<2>(d.c0, v) + chunk_pdot<2>(d.c1, v + ST), vsum, d.s, d.b);
          } else {
            const Q4Mat& m = e >= 0 ? p.L.down : p.L.sh_down;
            const int64_t oc = e >= 0 ? e * mat_codes : 0, og = e >= 0 ? e * mat_groups : 0;
            const uint4* cr = reinterpret_cast<const uint4*>(m.codes + oc) + (int64_t)n * CI;
            const uint16_t* sr = m.scales + og + (int64_t)n * GI;
            const uint16_t* br = m.biases + og + (int64_t)n * GI;
            for (int g = subI; g < GI; g += LI) {
              const uint4 c0 = cr[2 * g], c1 = cr[2 * g + 1];
              const uint32_t* v = ap + ((size_t)j * CI + 2 * g) * ST;
              const float vsum = as[j * CI + 2 * g] + as[j * CI + 2 * g + 1];
              part += affine_term(chunk_pdot<2>(c0, v) + chunk_pdot<2>(c1, v + ST), vsum, sr[g], br[g]);
            }
          }
          acc = fmaf(s_w[j], part, acc);
        }
      }
      acc = group_sum_rt(acc, p.lsI);
      if (subI == 0) s_red[wv][rsubI] = acc;
      __syncthreads();
      if (wv == 0 && lane < rpiI) {
        const int nn = rb * rpiI + lane;
        if (nn < H) {
          float t = s_red[0][lane];
#pragma unroll
          for (int w = 1; w < kWaves; ++w) t += s_red[w][lane];
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.y)[nn] = (uint16_t)f32_to_bf16_bits(t);
          else
            reinterpret_cast<float*>(p.y)[nn] = t;
        }
      }
      __syncthreads();
    }
  }
}

int lanes_log2(int groups) {
  int r = 0;
  while (r < 6 && (2 << r) <= groups) ++r;
  return r;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t decode_lds(const DecodeLayer& L) {
  const int nslot = L.top_k + (L.has_shared ? 1 : 0);
  return (size_t)(L.hidden >> 5) * (chunk_stride<1>() * 4 + 4) +
         (size_t)nslot * (L.inter >> 5) * (chunk_stride<2>() * 4 + 4);
}

}  // namespace

size_t decode_workspace_bytes(int hidden, int inter, int n_experts, int top_k) {
  (void)hidden;
  (void)n_experts;
  return align256(sizeof(DecodeWs)) + align256((size_t)(top_k + 1) * inter * 4);
}

size_t decode_lds_bytes(const DecodeLayer& L) { return decode_lds(L); }

hipError_t run_moe_ffn_decode(const DecodeLayer& L, const uint16_t* x, void* y, int out_bf16, int32_t* ids_out,
                              float* w_out, void* ws, hipStream_t stream) {
  DecodeParams p{};
  p.L = L;
  p.x = x;
  p.y = y;
  p.out_bf16 = out_bf16;
  p.ids_out = ids_out;
  p.w_out = w_out;
  char* w = static_cast<char*>(ws);
  p.ws = reinterpret_cast<DecodeWs*>(w);
  w += align256(sizeof(DecodeWs));
  p.act = reinterpret_cast<float*>(w);
  p.lsH = lanes_log2(L.hidden / kGroup);
  p.lsI = lanes_log2(L.inter / kGroup);
  const size_t lds = decode_lds(L);
  int blocks = device_cu_count();
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  hipLaunchKernelGGL(decode_layer_kernel, dim3(blocks), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace q4moe
