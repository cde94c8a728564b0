// Batched decode of one MoE feed-forward layer: B = 1..8 tokens, one per
// request, decoded together (lily-qwen3.8-flash-next, "Running it": several
// requests, four by default, decode in one step).
//
// Two launches on one stream:
//   1 front (one workgroup per CU, all resident together): every workgroup
//     dots its router row(s) with every token and publishes the logits as
//     epoch-tagged words (handoff.h); wave b then takes token b's top-k from
//     the published logits, and every workgroup builds the same plan: the
//     distinct experts named, in ascending id, then the shared expert, and per
//     planned expert the slot of each token that chose it.  The gate/up row
//     pairs of the planned experts are then spread over every wave of the grid
//     (a wave takes one row pair, its 64 lanes a 32-column chunk each, with
//     the next row pairs' loads in flight); each pair is dotted with the x of
//     each token that chose the expert, and the SwiGLU outputs go to
//     act[b][slot][i] (fp32).  Workgroup 0 writes the plan and the weights.
//   2 down: a workgroup owns 8 output rows for a subset of the tokens; its
//     waves issue the down-row loads of the planned experts those tokens
//     chose, the SwiGLU outputs are staged exactly as hi/lo bfloat16 pairs, and
//     each expert's rows are dotted with every token that chose it; the waves'
//     partial sums are added in a fixed order.
// The weights are read once per step whatever the number of tokens sharing an
// expert, which is what batching buys on a bandwidth-bound step.
#include <algorithm>
#include <mutex>

#include "handoff.h"
#include "kernels.h"
#include "topk.h"
#include "vecstage.h"

namespace q4moe {

namespace {

constexpr int kBitWords = kMaxExperts / 32;
static_assert(kBitWords <= kWave, "one bitmap word per lane of a wave");
constexpr int kMaxPlan = kMaxBatch * kMaxTopK + 1;  // distinct experts of a step, shared one included
constexpr int kFrontThreads = 512;             // front launch
constexpr int kFrontWaves = kFrontThreads / kWave;
constexpr int kFrontSlots = 4;                 // gate/up row pairs per wave whose loads are in flight together
constexpr int kLogitCopies = 8;                // copies of the tagged logits (workgroup b reads copy b % 8)

// The step's plan, built by every front workgroup and written out by workgroup 0.
struct BatchPlan {
  int n;                                // planned experts (distinct routed ones, then the shared one)
  int n_routed;
  int32_t expert[kMaxPlan];             // ascending routed ids, then -1 for the shared expert
  alignas(8) int8_t slot[kMaxPlan][kMaxBatch];  // slot of token b that chose planned expert d, or -1
};

// Head of the workspace: the front launch's epoch counters (timeout count at byte
// 2048) and its tagged logits, logit (token b, expert e) at word b * E + e of a copy.
struct FrontWs {
  HandoffHead h;
  unsigned long long tag_logit[kLogitCopies][kMaxBatch * kMaxExperts];
};

struct BatchParams {
  DecodeLayer L;
  const uint16_t* X;  // [B][H]
  int B;
  FrontWs* fws;
  BatchPlan* plan;
  float* wts;         // [B][k+1]: routing weights, then the shared expert's weight
  float* act;         // [B][nslot]: I / 32 chunk images of 32 words (16 hi, 16 lo bf16 pair words)
  void* y;            // [B][H]
  int out_bf16;
  int32_t* ids_out;   // nullable [B][k]
  float* w_out;       // nullable [B][k]
  int tpp;            // tokens per down workgroup
};

// Phase stamps of the front launch, in the diagnostic build only (-DQ4MOE_DECODE_STAMPS):
// thread 0 of every workgroup records the 100 MHz s_memrealtime counter, slot (epoch % 4)
// of the array (q4moe_front_stamps below): 0 launch start, 1 router logits published,
// 2 x staged, 3 top-k known, 4 plan ready, 5 end.
#ifdef Q4MOE_DECODE_STAMPS
constexpr int kStampBlocks = 1024;
__device__ unsigned long long g_front_stamps[4][kStampBlocks][8];
// the down launch's: 0 launch start, 1 plan in LDS, 2 task list built, 3 activations staged,
// 4 dots done, 5 end (slot: the front launch's epoch % 4; workgroup blockIdx.x of pass 0)
__device__ unsigned long long g_down_stamps[4][kStampBlocks][8];
#define Q4MOE_FSTAMP(i, v)                                                                        \
  do {                                                                                            \
    if (threadIdx.x == 0 && blockIdx.x < kStampBlocks) g_front_stamps[s_epoch & 3][blockIdx.x][i] = (v); \
  } while (0)
#else
#define Q4MOE_FSTAMP(i, v) \
  do {                     \
  } while (0)
#endif

// ---------------------------------------------------------------- launch 1
// One gate/up row pair: this lane's 32-column chunk of each row (4-bit: 16 bytes;
// 8-bit shared rows: 32 bytes, g/g2 and u/u2) and the chunk's group scale and bias.
struct GuRegs {
  uint4 g, u, g2, u2;
  uint32_t gs, gb, us, ub;
};

template <int NB, bool kLong>
__device__ __forceinline__ void batch_front(const BatchParams& p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ int32_t s_id[kMaxBatch][kMaxTopK];
  __shared__ float s_w[kMaxBatch][kMaxTopK];
  __shared__ float s_rpart[kMaxBatch][kFrontWaves];
  __shared__ uint32_t s_bits[kBitWords];
  __shared__ int s_pre[kBitWords + 1];
  __shared__ alignas(8) int8_t s_slot[kMaxPlan][kMaxBatch];
  __shared__ int32_t s_expert[kMaxPlan];
  __shared__ uint32_t s_epoch;

  const DecodeLayer& L = p.L;
  const int H = L.hidden, I = L.inter, E = L.n_experts, k = L.top_k;
  const int CH = H >> 5, G = H >> 6;
  // (the wave index read through a scalar register: the compiler then knows every task
  // index below is wave-uniform, so the branches on them stay scalar)
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), t = threadIdx.x;
  const int NBk = gridDim.x, b = blockIdx.x;
  FrontWs* ws = p.fws;
  constexpr int ST = chunk_stride<1>();
  uint32_t* xp = smem;                                              // [NB][CH][ST] x as permuted bf16 pairs
  float* xs = reinterpret_cast<float*>(xp + (size_t)NB * CH * ST);  // [NB][CH] chunk sums

  unsigned long long arrival = 0;
  if (t == 0) arrival = epoch_arrive(&ws->h, b);
#ifdef Q4MOE_DECODE_STAMPS
  const unsigned long long stamp0 = __builtin_amdgcn_s_memrealtime();
#endif

  // ---- A: router rows e = b, b + NBk, ... dotted with every token, published as tagged words
  const int nrows = b < E ? (E - 1 - b) / NBk + 1 : 0;
  for (int m = 0; m < nrows; ++m) {
    const int e = b + m * NBk;
    float acc[NB];
#pragma unroll
    for (int tok = 0; tok < NB; ++tok) acc[tok] = 0.f;
    if (L.router_q8.codes) {  // 8-bit router: 16-code chunks, each inside one 64-column group
      const uint4* r = reinterpret_cast<const uint4*>(L.router_q8.codes) + (size_t)e * (H >> 4);
      for (int c = t; c < (H >> 4); c += kFrontThreads) {
        const uint4 w = r[c];
        const float sc = bf16_bits_to_f32(L.router_q8.scales[(size_t)e * G + (c >> 2)]);
        const float bi = bf16_bits_to_f32(L.router_q8.biases[(size_t)e * G + (c >> 2)]);
        const uint32_t cw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int tok = 0; tok < NB; ++tok) {
          const uint4 xa = reinterpret_cast<const uint4*>(p.X + (size_t)tok * H)[2 * c];
          const uint4 xb = reinterpret_cast<const uint4*>(p.X + (size_t)tok * H)[2 * c + 1];
          const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
          float pq = 0.f, xsum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float xi = bf16_bits_to_f32((xw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
            xsum += xi;
            pq = fmaf(xi, (float)((cw[i >> 2] >> (8 * (i & 3))) & 0xFFu), pq);
          }
          acc[tok] += fmaf(sc, pq, bi * xsum);
        }
      }
    } else {
      const uint4* r = reinterpret_cast<const uint4*>(L.router) + (size_t)e * (H >> 3);
      for (int c = t; c < (H >> 3); c += kFrontThreads) {
        const uint4 w = r[c];
#pragma unroll
        for (int tok = 0; tok < NB; ++tok) {
          const uint4 v = reinterpret_cast<const uint4*>(p.X + (size_t)tok * H)[c];
          acc[tok] = dot2_bf16(w.w, v.w, dot2_bf16(w.z, v.z, dot2_bf16(w.y, v.y, dot2_bf16(w.x, v.x, acc[tok]))));
        }
      }
    }
#pragma unroll
    for (int tok = 0; tok < NB; ++tok) {
      const float r = group_sum_rt(acc[tok], 6);
      if (lane == 0) s_rpart[tok][wv] = r;
    }
    if (t == 0 && m == 0) s_epoch = epoch_finish(&ws->h, b, NBk, arrival);
    lds_sync();
    if (t < NB * kLogitCopies) {  // one thread per (token, copy); the waves' partials in a fixed order
      const int tok = t / kLogitCopies, c = t % kLogitCopies;
      float v = s_rpart[tok][0];
#pragma unroll
      for (int w = 1; w < kFrontWaves; ++w) v += s_rpart[tok][w];
      __hip_atomic_store(&ws->tag_logit[c][(size_t)tok * E + e], tag_word(s_epoch, v), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    lds_sync();  // s_rpart is reused
  }
  if (t == 0 && nrows == 0) s_epoch = epoch_finish(&ws->h, b, NBk, arrival);
#ifdef Q4MOE_DECODE_STAMPS
  Q4MOE_FSTAMP(0, stamp0);  // (thread 0 wrote s_epoch itself)
  Q4MOE_FSTAMP(1, __builtin_amdgcn_s_memrealtime());
#endif
  // x of every token, for the gate/up dots (while the other workgroups' logits arrive)
  for (int i = t; i < NB * CH; i += kFrontThreads) {
    const int tok = i / CH, c = i - tok * CH;
    stage_bf16_chunk(p.X + (size_t)tok * H, c, xp + (size_t)i * ST, xs + i);
  }
  lds_sync();
  const uint32_t epoch = s_epoch;
  Q4MOE_FSTAMP(2, __builtin_amdgcn_s_memrealtime());

  // ---- B: wave tok takes token tok's top-k (and its shared-expert weight)
  if (wv < NB) {
    const int tok = wv;
    float sw = 1.0f;
    if (L.sh_gate_w) {  // sigmoid(sh_gate_w . x)
      const uint4* gw = reinterpret_cast<const uint4*>(L.sh_gate_w);
      const uint4* gx = reinterpret_cast<const uint4*>(p.X + (size_t)tok * H);
      float d0 = 0.f, d1 = 0.f;
      for (int c = lane; c < (H >> 3); c += kWave) {
        const uint4 a = gw[c], x = gx[c];
        d0 = dot2_bf16(a.x, x.x, d0);
        d1 = dot2_bf16(a.y, x.y, d1);
        d0 = dot2_bf16(a.z, x.z, d0);
        d1 = dot2_bf16(a.w, x.w, d1);
      }
      sw = 1.0f / (1.0f + __expf(-group_sum_rt(d0 + d1, 6)));
    }
    const unsigned long long* tags = ws->tag_logit[b % kLogitCopies] + (size_t)tok * E;
    int32_t* io = b == 0 && p.ids_out ? p.ids_out + tok * k : nullptr;
    float* wo = b == 0 && p.w_out ? p.w_out + tok * k : nullptr;
    if (E <= 4 * kWave)
      wave_topk_tagged<4, 1>(tags, E, k, epoch, &ws->h.timeouts, s_id[tok], s_w[tok], io, wo);
    else if (E <= 8 * kWave)
      wave_topk_tagged<8, 1>(tags, E, k, epoch, &ws->h.timeouts, s_id[tok], s_w[tok], io, wo);
    else
      wave_topk_tagged<kMaxExperts / kWave, 1>(tags, E, k, epoch, &ws->h.timeouts, s_id[tok], s_w[tok], io, wo);
    if (b == 0) {
      if (lane < k) p.wts[tok * (k + 1) + lane] = s_w[tok][lane];
      if (lane == 0) p.wts[tok * (k + 1) + k] = sw;
    }
  }
  // ---- the plan (every workgroup alike): distinct experts ranked by id through a bitmap
  for (int i = t; i < kBitWords; i += kFrontThreads) s_bits[i] = 0u;
  lds_sync();
  Q4MOE_FSTAMP(3, __builtin_amdgcn_s_memrealtime());
  for (int i = t; i < NB * k; i += kFrontThreads) {
    const int id = s_id[i / k][i % k];
    atomicOr(&s_bits[id >> 5], 1u << (id & 31));
  }
  lds_sync();
  if (wv == 0) {  // exclusive prefix of the per-word counts (at most 32), from six bit-plane ballots
    const int c = lane < kBitWords ? __popc(s_bits[lane]) : 0;
    int before = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t plane = __ballot((c >> bit) & 1);
      before += __builtin_amdgcn_mbcnt_hi((uint32_t)(plane >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)plane, 0u)) << bit;
      total += __popcll(plane) << bit;
    }
    if (lane < kBitWords) s_pre[lane] = before;
    if (lane == 0) s_pre[kBitWords] = total;
  }
  lds_sync();
  const int nd = s_pre[kBitWords];
  const int n = nd + (L.has_shared ? 1 : 0);
  for (int i = t; i < n * kMaxBatch; i += kFrontThreads) {
    const int d = i / kMaxBatch, tok = i - d * kMaxBatch;
    s_slot[d][tok] = (int8_t)(d == nd && tok < NB ? k : -1);  // the shared expert serves every token
    if (tok == 0 && d == nd) s_expert[d] = -1;
  }
  lds_sync();
  for (int i = t; i < NB * k; i += kFrontThreads) {
    const int tok = i / k, j = i - tok * k, id = s_id[tok][j];
    const int d = s_pre[id >> 5] + __popc(s_bits[id >> 5] & ((1u << (id & 31)) - 1u));
    s_slot[d][tok] = (int8_t)j;
    s_expert[d] = id;  // every token naming the expert writes the same value
  }
  lds_sync();
  if (b == 0) {
    BatchPlan* plan = p.plan;
    for (int i = t; i < n * kMaxBatch; i += kFrontThreads)
      plan->slot[i / kMaxBatch][i % kMaxBatch] = s_slot[i / kMaxBatch][i % kMaxBatch];
    for (int i = t; i < n; i += kFrontThreads) plan->expert[i] = s_expert[i];
    if (t == 0) {
      plan->n = n;
      plan->n_routed = nd;
    }
  }

  Q4MOE_FSTAMP(4, __builtin_amdgcn_s_memrealtime());
  // ---- C: gate/up row pairs tau = d * I + i over every wave of the grid, pass q taking
  // tau = (q * NBk + b) * waves + wave; each wave keeps kFrontSlots passes of loads in
  // flight.  4-bit experts (routed, and a 4-bit shared one) take that pipelined loop; an
  // 8-bit shared expert's rows (plan entry nd) are spread over the waves the same way,
  // one pass at a time.
  const int nslot = k + (L.has_shared ? 1 : 0);
  const bool q8sh = L.has_shared && L.sh_q8;
  const int ntask = (q8sh ? nd : n) * I;  // 4-bit row pairs
  const int per_pass = NBk * kFrontWaves;
  const int npass = (ntask + per_pass - 1) / per_pass;
  const int64_t mat_codes = (int64_t)I * (H >> 3), mat_groups = (int64_t)I * G;
  const int c0 = min(lane, CH - 1);  // this lane's first chunk (lanes past CH: a valid chunk, not used)
  auto task_of = [&](int q) { return (q * NBk + b) * kFrontWaves + wv; };
  // this lane's chunk c of row pair (d, i) of a 4-bit expert (routed, or the shared one)
  auto load_chunk = [&](int d, int i, int c) __attribute__((always_inline)) {
    GuRegs r;
    const int e = __builtin_amdgcn_readfirstlane(s_expert[d]);
    const int64_t oc = e >= 0 ? e * mat_codes : 0, og = e >= 0 ? e * mat_groups : 0;
    const uint32_t* gc = e >= 0 ? L.gate.codes : L.sh_gate.codes;
    const uint32_t* uc = e >= 0 ? L.up.codes : L.sh_up.codes;
    const uint16_t* gsp = e >= 0 ? L.gate.scales : L.sh_gate.scales;
    const uint16_t* gbp = e >= 0 ? L.gate.biases : L.sh_gate.biases;
    const uint16_t* usp = e >= 0 ? L.up.scales : L.sh_up.scales;
    const uint16_t* ubp = e >= 0 ? L.up.biases : L.sh_up.biases;
    r.g = reinterpret_cast<const uint4*>(gc + oc + (int64_t)i * (H >> 3))[c];
    r.u = reinterpret_cast<const uint4*>(uc + oc + (int64_t)i * (H >> 3))[c];
    r.g2 = r.g;
    r.u2 = r.u;
    r.gs = gsp[og + (int64_t)i * G + (c >> 1)];
    r.gb = gbp[og + (int64_t)i * G + (c >> 1)];
    r.us = usp[og + (int64_t)i * G + (c >> 1)];
    r.ub = ubp[og + (int64_t)i * G + (c >> 1)];
    return r;
  };
  // the same for the 8-bit shared expert's row pair i: 32 code bytes per chunk
  auto load_chunk8 = [&](int i, int c) __attribute__((always_inline)) {
    GuRegs r;
    const uint4* gq = reinterpret_cast<const uint4*>(L.sh_gate.codes) + (int64_t)i * (H >> 4) + 2 * c;
    const uint4* uq = reinterpret_cast<const uint4*>(L.sh_up.codes) + (int64_t)i * (H >> 4) + 2 * c;
    r.g = gq[0];
    r.g2 = gq[1];
    r.u = uq[0];
    r.u2 = uq[1];
    r.gs = L.sh_gate.scales[(int64_t)i * G + (c >> 1)];
    r.gb = L.sh_gate.biases[(int64_t)i * G + (c >> 1)];
    r.us = L.sh_up.scales[(int64_t)i * G + (c >> 1)];
    r.ub = L.sh_up.biases[(int64_t)i * G + (c >> 1)];
    return r;
  };
  // row pair (d, i) against the x of each token that chose expert d; SwiGLU into act
  auto compute_pair = [&](int d, int i, const GuRegs r0, bool q8) __attribute__((always_inline)) {
    uint2 sl = *reinterpret_cast<const uint2*>(&s_slot[d][0]);
    sl.x = __builtin_amdgcn_readfirstlane(sl.x);
    sl.y = __builtin_amdgcn_readfirstlane(sl.y);
    auto slot_of = [&](int tok) { return (int)(int8_t)(((tok < 4 ? sl.x : sl.y) >> (8 * (tok & 3))) & 0xFFu); };
    float ag[NB], au[NB];
#pragma unroll
    for (int tok = 0; tok < NB; ++tok) ag[tok] = au[tok] = 0.f;
    auto accumulate = [&](const GuRegs& r, int c) __attribute__((always_inline)) {
#pragma unroll
      for (int tok = 0; tok < NB; ++tok) {
        if (slot_of(tok) < 0) continue;  // (uniform over the wave)
        const uint32_t* v = xp + ((size_t)tok * CH + c) * ST;
        const float vs = xs[tok * CH + c];
        if (q8) {  // w = s q + b
          ag[tok] += fmaf(bf16_bits_to_f32(r.gs), q8_chunk_pdot<1>(r.g, r.g2, v), bf16_bits_to_f32(r.gb) * vs);
          au[tok] += fmaf(bf16_bits_to_f32(r.us), q8_chunk_pdot<1>(r.u, r.u2, v), bf16_bits_to_f32(r.ub) * vs);
        } else {
          ag[tok] += affine_term(chunk_pdot<1>(r.g, v), vs, r.gs, r.gb);
          au[tok] += affine_term(chunk_pdot<1>(r.u, v), vs, r.us, r.ub);
        }
      }
    };
    if (lane < CH) accumulate(r0, lane);
    // rows longer than 2048 columns (kLong): the further chunks, loaded here (a loop that
    // loads makes the compiler wait for every load in flight at its head, so the form
    // for rows of at most 2048 columns has none)
    if constexpr (kLong)
      for (int c = lane + kWave; c < CH; c += kWave) accumulate(q8 ? load_chunk8(i, c) : load_chunk(d, i, c), c);
#pragma unroll
    for (int tok = 0; tok < NB; ++tok) {
      const int j = slot_of(tok);
      if (j < 0) continue;
      const float g = group_sum_rt(ag[tok], 6), u = group_sum_rt(au[tok], 6);
      if (lane == 0) {  // into the staged image: hi/lo bf16 parts at the permuted pair positions
        const float a = silu(g) * u;
        const uint32_t hb = f32_to_bf16_bits(a), lb = f32_to_bf16_bits(a - bf16_bits_to_f32(hb));
        uint16_t* img = reinterpret_cast<uint16_t*>(p.act) + ((size_t)(tok * nslot + j) * I + (i & ~31)) * 2;
        const int w = i & 7, off = (4 * ((i & 31) >> 3) + (w & 3)) * 2 + (w >> 2);
        img[off] = (uint16_t)hb;
        img[off + 32] = (uint16_t)lb;
      }
    }
  };
  // loads are issued unconditionally (a task past the end reads the last valid row pair,
  // unused): a load behind a branch makes the compiler wait for every load in flight
  const int last = max(ntask - 1, 0);
  GuRegs rr[kFrontSlots];
#pragma unroll
  for (int s = 0; s < kFrontSlots; ++s) {
    const int tau = min(task_of(s), last);
    rr[s] = load_chunk(tau / I, tau % I, c0);
  }
  if (q8sh) {  // the 8-bit shared expert's row pairs, loaded behind the first 4-bit passes
    for (int q = 0;; ++q) {
      const int i = task_of(q);
      if (i >= I) break;
      compute_pair(nd, i, load_chunk8(i, c0), true);
    }
  }
  for (int q0 = 0; q0 < npass; q0 += kFrontSlots) {
#pragma unroll
    for (int s = 0; s < kFrontSlots; ++s) {
      const int tau = task_of(q0 + s), tau2 = min(task_of(q0 + s + kFrontSlots), last);
      if (tau < ntask) compute_pair(tau / I, tau % I, rr[s], false);
      rr[s] = load_chunk(tau2 / I, tau2 % I, c0);
    }
  }
#ifdef Q4MOE_DECODE_STAMPS
  wait_vmem();  // (the activation stores are out)
  __syncthreads();  // every wave of the workgroup is done
  Q4MOE_FSTAMP(5, __builtin_amdgcn_s_memrealtime());
#endif
}

// NB tokens; kLong: hidden above 2048 (more than one 32-column chunk per lane)
#define Q4MOE_FRONT_KERNEL(NB)                                                                       \
  __global__ __launch_bounds__(kFrontThreads) void batch_front_kernel_##NB(BatchParams p) { batch_front<NB, false>(p); } \
  __global__ __launch_bounds__(kFrontThreads) void batch_front_long_kernel_##NB(BatchParams p) { batch_front<NB, true>(p); }
Q4MOE_FRONT_KERNEL(1)
Q4MOE_FRONT_KERNEL(2)
Q4MOE_FRONT_KERNEL(3)
Q4MOE_FRONT_KERNEL(4)
Q4MOE_FRONT_KERNEL(5)
Q4MOE_FRONT_KERNEL(6)
Q4MOE_FRONT_KERNEL(7)
Q4MOE_FRONT_KERNEL(8)
#undef Q4MOE_FRONT_KERNEL

// ---------------------------------------------------------------- launch 2
// Workgroup (x, y) owns output rows 8x .. 8x + 7 for tokens y*tpp .. of the pass.  The
// planned experts that a token of the pass chose are listed; each listed expert's 8 rows
// are kDownTPE tasks of 4 rows (16 lanes a row, one 32-column chunk a lane; an 8-bit shared
// row's chunk is 32 bytes), spread over the waves, and the loads of the first
// kDownSlots tasks of every wave are issued before the SwiGLU outputs are staged.  Each
// task writes the 4-row dot of every token of the pass that chose the expert to
// s_red[token][slot][row]; the output is the fixed-order weighted sum over the slots.
constexpr int kDownThreads = 1024;
constexpr int kDownWaves = kDownThreads / kWave;
constexpr int kDownSlots = 6;     // tasks per wave whose loads are issued ahead
constexpr int kDownRowLanes = 16;  // lanes per down row
constexpr int kDownTaskRows = kWave / kDownRowLanes;  // rows of one task
#ifndef Q4MOE_DOWN_ROWS
#define Q4MOE_DOWN_ROWS 8
#endif
constexpr int kDownRows = Q4MOE_DOWN_ROWS;  // output rows per workgroup
constexpr int kDownTPE = kDownRows / kDownTaskRows;  // tasks per (planned expert, token) entry
static_assert(kDownRows % kDownTaskRows == 0 && (kDownTPE & (kDownTPE - 1)) == 0, "whole tasks, a power of two");

struct DnRegs {
  uint4 c, c2;  // c2: the second 16 bytes of an 8-bit row's chunk (else c again)
  uint32_t s, b;
};

template <bool kLong>
__device__ __forceinline__ void batch_down(const BatchParams& p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ float s_w[kMaxBatch][kMaxTopK + 1];
  __shared__ float s_red[kMaxBatch][kMaxTopK + 1][kDownRows];
  __shared__ alignas(8) int8_t s_slot[kMaxPlan][kMaxBatch];
  __shared__ int32_t s_expert[kMaxPlan];
  __shared__ int16_t s_list[kMaxPlan * kMaxBatch];  // (planned expert << 3 | token of the pass)
  __shared__ int s_nlist;

  const DecodeLayer& L = p.L;
  const int H = L.hidden, I = L.inter, k = L.top_k;
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), t = threadIdx.x;
  const int b0 = blockIdx.y * p.tpp, nb = min(p.tpp, p.B - b0);
  const int n0 = blockIdx.x * kDownRows;
  const int nslot = k + (L.has_shared ? 1 : 0);
  const int GI = I >> 6, CI = I >> 5;
  const BatchPlan* plan = p.plan;
  const int nall = plan->n;
#ifdef Q4MOE_DECODE_STAMPS
  const unsigned long long dstamp0 = __builtin_amdgcn_s_memrealtime();
  const unsigned dslot = (unsigned)(p.fws->h.group_ctr[0][0] >> 32) & 3u;
  unsigned long long* dst = g_down_stamps[dslot][blockIdx.x < kStampBlocks ? blockIdx.x : 0];
  const bool dstamp = threadIdx.x == 0 && blockIdx.y == 0 && blockIdx.x < kStampBlocks;
#define Q4MOE_DSTAMP(i, v) \
  do {                     \
    if (dstamp) dst[i] = (v); \
  } while (0)
#else
#define Q4MOE_DSTAMP(i, v) \
  do {                     \
  } while (0)
#endif
  Q4MOE_DSTAMP(0, dstamp0);
  // The plan (every entry, used or not, so that these loads go out with the one of n) and
  // the routing weights into registers, then the SwiGLU output images of this pass's
  // tokens (they do not depend on the plan; the first chunk of each thread is loaded here,
  // so its latency overlaps the plan's), then the plan into LDS.
  static_assert(kMaxPlan <= kDownThreads && kMaxBatch == 8, "one plan row (8 bytes) per thread");
  const int nwt = nb * (k + 1);
  const int ip = min(t, kMaxPlan - 1), iw = min(t, nwt - 1);
  const int bw = iw / (k + 1), jw = iw - bw * (k + 1);
  const uint2* ps = reinterpret_cast<const uint2*>(&plan->slot[0][0]) + ip;
  const int32_t* pe = plan->expert + ip;
  const float* pwp = p.wts + (b0 + bw) * (k + 1) + jw;  // slot k: the shared expert's weight
  __builtin_amdgcn_sched_barrier(0);  // addresses first, then the three loads back to back
  const float pw = *pwp;
  const uint2 pslot = *ps;
  const int32_t pexp = *pe;
  __builtin_amdgcn_sched_barrier(0);  // the plan's loads go out first: its wait then excludes the images
  constexpr int ST = chunk_stride<2>();
  const int nchunk = nb * nslot * CI;
  const uint4* img = reinterpret_cast<const uint4*>(p.act) + (size_t)b0 * nslot * CI * 8;
  // Wave wv copies chunks 64 wv .. 64 wv + 63 (8 KB, contiguous) in eight 1 KB loads:
  // load q of lane l is 16-byte piece l % 8 of chunk 64 wv + 8q + l / 8.
  const int nw = nchunk * 8;  // 16-byte pieces of the images
  uint4 w0[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) w0[q] = img[min(wv * 512 + q * 64 + lane, nw - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // (unconditional: threads past the plan rewrite its last entry with the same value, so
  // no branch invites the compiler to sink the plan's loads behind the images')
  reinterpret_cast<uint2*>(&s_slot[0][0])[ip] = pslot;
  s_expert[ip] = pexp;
  s_w[bw][jw] = pw;
  lds_sync();
  Q4MOE_DSTAMP(1, __builtin_amdgcn_s_memrealtime());
  if (wv == 0) {  // (planned expert, token) for each token of the pass that chose it, in plan order
    int cnt = 0;
    for (int d0 = 0; d0 < nall; d0 += kWave) {
      const int dd = d0 + lane;
      uint32_t mine = 0;  // bit bb: token b0 + bb chose expert dd
      if (dd < nall) {
        const uint2 row = *reinterpret_cast<const uint2*>(&s_slot[dd][0]);  // slot bytes of tokens 0..7
        const uint64_t r64 = (uint64_t)row.y << 32 | row.x;
#pragma unroll
        for (int bb = 0; bb < kMaxBatch; ++bb)
          mine |= (bb < nb && (int8_t)((r64 >> (8 * ((b0 + bb) & 7))) & 0xFFu) >= 0 ? 1u : 0u) << bb;
      }
      // exclusive prefix of the counts (at most 8) over the lanes, from four bit-plane ballots
      const int c = __popc(mine);
      int before = 0, total = 0;
#pragma unroll
      for (int bit = 0; bit < 4; ++bit) {
        const uint64_t plane = __ballot((c >> bit) & 1);
        before += __builtin_amdgcn_mbcnt_hi((uint32_t)(plane >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)plane, 0u)) << bit;
        total += __popcll(plane) << bit;
      }
      int at = cnt + before;
      for (uint32_t m = mine; m; m &= m - 1) s_list[at++] = (int16_t)(dd << 3 | __builtin_ctz(m));
      cnt += total;
    }
    if (lane == 0) s_nlist = cnt;
  }
  lds_sync();
  Q4MOE_DSTAMP(2, __builtin_amdgcn_s_memrealtime());
  // task tau: entry tau / kDownTPE of the list, rows (tau % kDownTPE) * 4 + rsub of the block
  const int ntask = kDownTPE * s_nlist;
  const int last = max(ntask - 1, 0);
  const int sub = lane & (kDownRowLanes - 1), rsub = lane / kDownRowLanes;
  const int c0 = min(sub, CI - 1);  // this lane's first chunk (lanes past CI: a valid chunk, not used)
  const bool q8sh = L.has_shared && L.sh_q8;
  const int64_t mat_codes = (int64_t)H * (I >> 3), mat_groups = (int64_t)H * GI;
  // (loads branch-free)
  auto load_dn = [&](int tau, int c) __attribute__((always_inline)) {
    DnRegs r;
    const int e = __builtin_amdgcn_readfirstlane(s_expert[s_list[tau / kDownTPE] >> 3]);
    const int n = min(n0 + (tau % kDownTPE) * kDownTaskRows + rsub, H - 1);
    const bool q8 = e < 0 && q8sh;
    const uint32_t* codes = e >= 0 ? L.down.codes + e * mat_codes : L.sh_down.codes;
    const uint16_t* sc = e >= 0 ? L.down.scales + e * mat_groups : L.sh_down.scales;
    const uint16_t* bi = e >= 0 ? L.down.biases + e * mat_groups : L.sh_down.biases;
    const uint4* cr = reinterpret_cast<const uint4*>(codes + (int64_t)n * (q8 ? I >> 2 : I >> 3)) + (q8 ? 2 * c : c);
    r.c = cr[0];
    r.c2 = cr[q8 ? 1 : 0];
    r.s = sc[(int64_t)n * GI + (c >> 1)];
    r.b = bi[(int64_t)n * GI + (c >> 1)];
    return r;
  };
  // stage the SwiGLU outputs of this pass's tokens, [nb][nslot] x ([CI][ST2] pairs, [CI]
  // sums): the chunk images are copied; a chunk's sum is the dot of its 32 words with
  // (1, 1).  The first chunk of each thread was loaded before the weight rows (its wait
  // then does not include theirs), the rest after.
  constexpr uint32_t kOnes = 0x3F803F80u;  // two bfloat16 1.0
  uint32_t* ap = smem;
  float* as = reinterpret_cast<float*>(ap + (size_t)p.tpp * nslot * CI * ST);
  DnRegs dr[kDownSlots];
#pragma unroll
  for (int q = 0; q < kDownSlots; ++q) dr[q] = load_dn(min(q * kDownWaves + wv, last), c0);
  // pieces of chunks c0w + 8q + lane / 8 into LDS; a chunk's sum meets in its 8 lanes
  auto put = [&](int c0w, const uint4 (&w)[8]) __attribute__((always_inline)) {
    const int pc = lane & 7;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = c0w + 8 * q + (lane >> 3);
      const float part = dot2_bf16(w[q].x, kOnes, dot2_bf16(w[q].y, kOnes, 0.f)) +
                         dot2_bf16(w[q].z, kOnes, dot2_bf16(w[q].w, kOnes, 0.f));
      const float sum = group_sum<8>(part);
      if (c < nchunk) {
        *reinterpret_cast<uint4*>(ap + (size_t)c * ST + 4 * pc) = w[q];
        if (pc == 0) as[c] = sum;
      }
    }
  };
  put(wv * 64, w0);
  for (int c0w = kDownThreads + wv * 64; c0w < nchunk; c0w += kDownThreads) {  // (more than 1,024 chunks)
    uint4 w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = img[min(c0w * 8 + q * 64 + lane, nw - 1)];
    put(c0w, w);
  }
  lds_sync();  // (an LDS-only barrier: the weight loads stay in flight)
  Q4MOE_DSTAMP(3, __builtin_amdgcn_s_memrealtime());

  auto compute = [&](int tau, const DnRegs r0) __attribute__((always_inline)) {
    const int ent = __builtin_amdgcn_readfirstlane(s_list[tau / kDownTPE]);
    const int dd = ent >> 3, bb = ent & 7;
    const bool q8 = __builtin_amdgcn_readfirstlane(s_expert[dd]) < 0 && q8sh;
    const int j = __builtin_amdgcn_readfirstlane(s_slot[dd][b0 + bb]);
    auto dot = [&](const DnRegs r, int c, int vi) __attribute__((always_inline)) {
      const uint32_t* v = ap + (size_t)vi * ST;
      return q8 ? fmaf(bf16_bits_to_f32(r.s), q8_chunk_pdot<2>(r.c, r.c2, v), bf16_bits_to_f32(r.b) * as[vi])
                : affine_term(chunk_pdot<2>(r.c, v), as[vi], r.s, r.b);
    };
    const int r = (tau % kDownTPE) * kDownTaskRows + rsub;
    const int vi = (bb * nslot + j) * CI;
    float part = sub < CI ? dot(r0, sub, vi + sub) : 0.f;
    if constexpr (kLong)  // rows of more than 16 chunks: the further chunks, loaded here
      for (int c = sub + kDownRowLanes; c < CI; c += kDownRowLanes) part += dot(load_dn(tau, c), c, vi + c);
    part = group_sum_rt(part, 4);
    if (sub == 0) s_red[bb][j][r] = part;
  };
  const int npass = (ntask + kDownWaves - 1) / kDownWaves;
#pragma unroll
  for (int q = 0; q < kDownSlots; ++q) {
    const int tau = q * kDownWaves + wv;
    if (tau < ntask) compute(tau, dr[q]);
  }
  for (int q = kDownSlots; q < npass; ++q) {  // (more tasks than the loads issued ahead)
    const int tau = q * kDownWaves + wv;
    const DnRegs r = load_dn(min(tau, last), c0);
    if (tau < ntask) compute(tau, r);
  }
  lds_sync();
  Q4MOE_DSTAMP(4, __builtin_amdgcn_s_memrealtime());
  for (int i = t; i < nb * kDownRows; i += kDownThreads) {
    const int bb = i / kDownRows, r = i - bb * kDownRows, nn = n0 + r;
    if (nn >= H) continue;
    float acc = 0.f;
    for (int j = 0; j < nslot; ++j) acc = fmaf(s_w[bb][j], s_red[bb][j][r], acc);  // fixed slot order
    const size_t o = (size_t)(b0 + bb) * H + nn;
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.y)[o] = (uint16_t)f32_to_bf16_bits(acc);
    else
      reinterpret_cast<float*>(p.y)[o] = acc;
  }
#ifdef Q4MOE_DECODE_STAMPS
  wait_vmem();
  __syncthreads();  // every wave of the workgroup is done
  Q4MOE_DSTAMP(5, __builtin_amdgcn_s_memrealtime());
#endif
#undef Q4MOE_DSTAMP
}

__global__ __launch_bounds__(kDownThreads) void batch_down_kernel(BatchParams p) { batch_down<false>(p); }
__global__ __launch_bounds__(kDownThreads) void batch_down_long_kernel(BatchParams p) { batch_down<true>(p); }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t front_lds(const DecodeLayer& L, int B) {
  return (size_t)B * (L.hidden >> 5) * (chunk_stride<1>() * 4 + 4);
}

size_t down_lds_per_token(const DecodeLayer& L) {
  const int nslot = L.top_k + (L.has_shared ? 1 : 0);
  return (size_t)nslot * (L.inter >> 5) * (chunk_stride<2>() * 4 + 4);
}

typedef void (*FrontKernel)(BatchParams);

FrontKernel front_kernel_for(const DecodeLayer& L, int B) {
  const bool lng = L.hidden > 32 * kWave;
#define Q4MOE_FRONT_CASE(NB) \
  case NB: return lng ? batch_front_long_kernel_##NB : batch_front_kernel_##NB;
  switch (B) {
    Q4MOE_FRONT_CASE(1)
    Q4MOE_FRONT_CASE(2)
    Q4MOE_FRONT_CASE(3)
    Q4MOE_FRONT_CASE(4)
    Q4MOE_FRONT_CASE(5)
    Q4MOE_FRONT_CASE(6)
    Q4MOE_FRONT_CASE(7)
    default: return lng ? batch_front_long_kernel_8 : batch_front_kernel_8;
  }
#undef Q4MOE_FRONT_CASE
}

}  // namespace

size_t decode_batch_workspace_bytes(int n_experts, int top_k, int inter, int B) {
  (void)n_experts;
  return align256(sizeof(FrontWs)) + align256(sizeof(BatchPlan)) + align256((size_t)B * (top_k + 1) * 4) +
         align256((size_t)B * (top_k + 1) * inter * 4);
}

bool decode_batch_supported(const DecodeLayer& L, int B, size_t max_lds) {
  // the down launch needs room for at least one token's SwiGLU outputs
  return front_lds(L, B) <= max_lds && down_lds_per_token(L) <= max_lds;
}

// The front launch's workgroups wait on each other's logits, so one per CU must fit
// at once (registers and LDS); cached per device, batch size and LDS size.
bool decode_batch_fits(const DecodeLayer& L, int B) {
  struct Entry {
    int dev;
    FrontKernel k;
    size_t lds;
    bool ok;
  };
  static Entry cache[64];
  static int ncache = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const size_t lds = front_lds(L, B);
  const FrontKernel kern = front_kernel_for(L, B);
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < ncache; ++i)
    if (cache[i].dev == dev && cache[i].k == kern && cache[i].lds == lds) return cache[i].ok;
  int per_cu = 0;
  const bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                               kFrontThreads, lds) == hipSuccess &&
                  per_cu >= 1;
  if (ncache < 64) cache[ncache++] = Entry{dev, kern, lds, ok};
  return ok;
}

// Dynamic LDS the down launch may take on the current device: the device's per-workgroup
// limit less the kernel's static arrays (at least max_lds, the limit every launch takes);
// above 64 KB the kernels are told once per device.
size_t down_lds_limit(size_t max_lds) {
  static size_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return max_lds;
  if (cached[dev]) return cached[dev];
  int per_block = 0;
  size_t lim = max_lds;
  hipFuncAttributes fa{};
  if (hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
      hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(batch_down_long_kernel)) == hipSuccess &&
      (size_t)per_block > fa.sharedSizeBytes + max_lds) {
    const size_t want = (size_t)per_block - fa.sharedSizeBytes;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(batch_down_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)want) == hipSuccess &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(batch_down_long_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)want) == hipSuccess)
      lim = want;
  }
  (void)hipGetLastError();
  cached[dev] = lim;
  return lim;
}

hipError_t run_moe_ffn_decode_batch(const DecodeLayer& L, const uint16_t* X, int B, void* y, int out_bf16,
                                    int32_t* ids_out, float* w_out, void* ws, size_t max_lds, hipStream_t stream) {
  BatchParams p{};
  p.L = L;
  p.X = X;
  p.B = B;
  char* w = static_cast<char*>(ws);
  p.fws = reinterpret_cast<FrontWs*>(w);
  w += align256(sizeof(FrontWs));
  p.plan = reinterpret_cast<BatchPlan*>(w);
  w += align256(sizeof(BatchPlan));
  p.wts = reinterpret_cast<float*>(w);
  w += align256((size_t)B * (L.top_k + 1) * 4);
  p.act = reinterpret_cast<float*>(w);
  p.y = y;
  p.out_bf16 = out_bf16;
  p.ids_out = ids_out;
  p.w_out = w_out;
  const size_t per_tok = down_lds_per_token(L);
  p.tpp = (int)std::min<size_t>((size_t)B, down_lds_limit(max_lds) / per_tok);

  hipLaunchKernelGGL(front_kernel_for(L, B), dim3(device_cu_count()), dim3(kFrontThreads), front_lds(L, B), stream, p);
  const int passes = (B + p.tpp - 1) / p.tpp;
  hipLaunchKernelGGL((L.inter > 32 * kDownRowLanes ? batch_down_long_kernel : batch_down_kernel),
                     dim3((L.hidden + kDownRows - 1) / kDownRows, passes), dim3(kDownThreads), (size_t)p.tpp * per_tok,
                     stream, p);
  return hipGetLastError();
}

}  // namespace q4moe

#ifdef Q4MOE_DECODE_STAMPS
// Diagnostic build only: copy the front launch's phase stamps ([4][1024][8] uint64, slot
// epoch % 4, stamps as listed above) to host memory.
extern "C" int q4moe_front_stamps(void* host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(q4moe::g_front_stamps), bytes);
}
// The same for the down launch's stamps.
extern "C" int q4moe_down_stamps(void* host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(q4moe::g_down_stamps), bytes);
}
#endif
