// Batched decode of one MoE feed-forward layer: B = 1..8 tokens, one per
// request, decoded together (lily-qwen3.8-flash-next, "Running it": several
// requests, four by default, decode in one step).
//
// Four launches on one stream, each reading what the previous one wrote:
//   1 route: logits[b][e] for every token, each router row read once for all
//     tokens (one row per wave);
//   2 plan (one workgroup): the B top-k lists, the distinct experts they name
//     in ascending id, then the shared expert, and per planned expert the slot
//     of each token that chose it;
//   3 gate/up: a workgroup takes a 32-row block of one planned expert: its
//     weight loads are issued, the x of the tokens that chose the expert are
//     staged, and each row is dotted with each of them; SwiGLU outputs go to
//     act[b][slot][i] (fp32);
//   4 down: a workgroup owns 8 output rows for a subset of the tokens; its
//     waves issue the down-row loads of the planned experts those tokens
//     chose, the SwiGLU outputs are staged exactly as hi/lo bfloat16 pairs, and
//     each expert's rows are dotted with every token that chose it; the waves'
//     partial sums are added in a fixed order.
// The weights are read once per step whatever the number of tokens sharing an
// expert, which is what batching buys on a bandwidth-bound step.
#include <algorithm>

#include "kernels.h"
#include "topk.h"
#include "vecstage.h"

namespace q4moe {

namespace {

constexpr int kRouteWaves = 8;                 // one router row per wave; one wave per token for the top-k
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kGateUpRows = kWaves * 8;        // rows of one expert per gate/up workgroup (8 per wave)
constexpr int kDownLanes = 8;                  // lanes per down row (groups sub, sub + 8, ...)
constexpr int kDownRows = kWave / kDownLanes;  // output rows per down workgroup: one per lane octet
constexpr int kDownPrefetch = 4;               // experts per wave whose down rows are loaded ahead
constexpr int kBitWords = kMaxExperts / 32;
constexpr int kMaxPlan = kMaxBatch * kMaxTopK + 1;  // distinct experts of a step, shared one included

// The step's plan, written by batch_plan_kernel (one workgroup) after the router launch.
struct BatchPlan {
  int n;                                // planned experts (distinct routed ones, then the shared one)
  int n_routed;
  int32_t expert[kMaxPlan];             // ascending routed ids, then -1 for the shared expert
  alignas(8) int8_t slot[kMaxPlan][kMaxBatch];  // slot of token b that chose planned expert d, or -1
};

struct BatchParams {
  DecodeLayer L;
  const uint16_t* X;  // [B][H]
  int B;
  float* logits;      // [B][E]
  BatchPlan* plan;
  float* wts;         // [B][k+1]: routing weights, then the shared expert's weight
  float* act;         // [B][nslot][I]
  void* y;            // [B][H]
  int out_bf16;
  int32_t* ids_out;   // nullable [B][k]
  float* w_out;       // nullable [B][k]
  int tpp;            // tokens per down workgroup
};

// ---------------------------------------------------------------- launch 1
// Wave w of workgroup r: logits[b][8r + w] = router[8r + w] . X[b] for every b < NB; with
// kQ8 the router is the layer's 8-bit affine matrix (16-code chunks per lane, each inside
// one 64-column group: scale * sum(x q) + bias * sum(x)).
template <int NB, bool kQ8>
__global__ __launch_bounds__(kRouteWaves * kWave) void batch_route_kernel(BatchParams p) {
  const int H = p.L.hidden, E = p.L.n_experts;
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int e = blockIdx.x * kRouteWaves + wv;
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  if constexpr (kQ8) {
    const int G = H >> 6, er = min(e, E - 1);
    const uint4* r = reinterpret_cast<const uint4*>(p.L.router_q8.codes) + (size_t)er * (H >> 4);
    const uint16_t* sr = p.L.router_q8.scales + (size_t)er * G;
    const uint16_t* br = p.L.router_q8.biases + (size_t)er * G;
    for (int c = lane; c < (H >> 4); c += kWave) {
      const uint4 w = r[c];
      const float sc = bf16_bits_to_f32(sr[c >> 2]), bi = bf16_bits_to_f32(br[c >> 2]);
      const uint32_t cw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 xa = reinterpret_cast<const uint4*>(p.X + (size_t)b * H)[2 * c];
        const uint4 xb = reinterpret_cast<const uint4*>(p.X + (size_t)b * H)[2 * c + 1];
        const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        float pq = 0.f, xs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float xi = bf16_bits_to_f32((xw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
          xs += xi;
          pq = fmaf(xi, (float)((cw[i >> 2] >> (8 * (i & 3))) & 0xFFu), pq);
        }
        acc[b] += fmaf(sc, pq, bi * xs);
      }
    }
  } else {
  const uint4* r = reinterpret_cast<const uint4*>(p.L.router + (size_t)min(e, E - 1) * H);
  const int nc = H >> 3;  // 16-byte chunks per row
  constexpr int Q = 4;    // chunks per lane in flight
  for (int c0 = 0; c0 < nc; c0 += Q * kWave) {
    uint4 w[Q], v[NB][Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = c0 + q * kWave + lane;
      const bool ok = c < nc;
      w[q] = ok ? r[c] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        v[b][q] = ok ? reinterpret_cast<const uint4*>(p.X + (size_t)b * H)[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < Q; ++q)
        acc[b] = dot2_bf16(w[q].w, v[b][q].w,
                           dot2_bf16(w[q].z, v[b][q].z, dot2_bf16(w[q].y, v[b][q].y, dot2_bf16(w[q].x, v[b][q].x, acc[b]))));
  }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float l = group_sum_rt(acc[b], 6);
    if (lane == 0 && e < E) p.logits[(size_t)b * E + e] = l;
  }
}

// ---------------------------------------------------------------- launch 2
// One workgroup plans the step: wave b takes token b's top-k; the distinct
// experts named are ranked by id through a bitmap with per-word prefix counts;
// the plan (per planned expert its id and the slot of each token that chose
// it, the shared expert last) is built in LDS and written out once.
template <int NB, int V>
__global__ __launch_bounds__(kRouteWaves * kWave) void batch_plan_kernel(BatchParams p) {
  __shared__ int32_t s_id[kMaxBatch][kMaxTopK];
  __shared__ float s_w[kMaxBatch][kMaxTopK];
  __shared__ uint32_t s_bits[kBitWords];
  __shared__ int s_pre[kBitWords + 1];
  __shared__ int8_t s_slot[kMaxPlan][kMaxBatch];
  __shared__ int32_t s_expert[kMaxPlan];
  const int E = p.L.n_experts, k = p.L.top_k;
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  if (wv < NB) {
    const int b = wv;
    wave_topk_sorted<V>(p.logits + (size_t)b * E, E, k, s_id[b], s_w[b]);
    if (lane < k) {
      p.wts[b * (k + 1) + lane] = s_w[b][lane];
      if (p.ids_out) p.ids_out[b * k + lane] = s_id[b][lane];
      if (p.w_out) p.w_out[b * k + lane] = s_w[b][lane];
    }
    // the shared expert's weight: 1, or sigmoid(sh_gate_w . x_b) when the layer has the gate
    float sw = 1.0f;
    if (p.L.sh_gate_w) {
      const int H = p.L.hidden;
      const uint4* gw = reinterpret_cast<const uint4*>(p.L.sh_gate_w);
      const uint4* gx = reinterpret_cast<const uint4*>(p.X + (size_t)b * H);
      float d0 = 0.f, d1 = 0.f;
      for (int c = lane; c < (H >> 3); c += kWave) {
        const uint4 a = gw[c], x = gx[c];
        d0 = dot2_bf16(a.x, x.x, d0);
        d1 = dot2_bf16(a.y, x.y, d1);
        d0 = dot2_bf16(a.z, x.z, d0);
        d1 = dot2_bf16(a.w, x.w, d1);
      }
      const float d = group_sum_rt(d0 + d1, 6);
      sw = 1.0f / (1.0f + __expf(-d));
    }
    if (lane == 0) p.wts[b * (k + 1) + k] = sw;
  }
  for (int i = threadIdx.x; i < kBitWords; i += blockDim.x) s_bits[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < NB * k; i += blockDim.x) {
    const int id = s_id[i / k][i % k];
    atomicOr(&s_bits[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  if (wv == 0) {  // exclusive prefix of the per-word counts
    const int c = lane < kBitWords ? __popc(s_bits[lane]) : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane < kBitWords) s_pre[lane] = incl - c;
    if (lane == kWave - 1) s_pre[kBitWords] = incl;
  }
  __syncthreads();
  const int nd = s_pre[kBitWords];
  const int n = nd + (p.L.has_shared ? 1 : 0);
  for (int i = threadIdx.x; i < n * kMaxBatch; i += blockDim.x) {
    const int d = i / kMaxBatch, b = i - d * kMaxBatch;
    s_slot[d][b] = (int8_t)(d == nd && b < NB ? k : -1);  // the shared expert serves every token with weight 1
    if (b == 0 && d == nd) s_expert[d] = -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NB * k; i += blockDim.x) {
    const int b = i / k, j = i - b * k, id = s_id[b][j];
    const int d = s_pre[id >> 5] + __popc(s_bits[id >> 5] & ((1u << (id & 31)) - 1u));
    s_slot[d][b] = (int8_t)j;
    s_expert[d] = id;  // every token naming the expert writes the same value
  }
  __syncthreads();
  BatchPlan* plan = p.plan;
  for (int i = threadIdx.x; i < n * kMaxBatch; i += blockDim.x)
    plan->slot[i / kMaxBatch][i % kMaxBatch] = s_slot[i / kMaxBatch][i % kMaxBatch];
  for (int i = threadIdx.x; i < n; i += blockDim.x) plan->expert[i] = s_expert[i];
  if (threadIdx.x == 0) {
    plan->n = n;
    plan->n_routed = nd;
  }
}

// ---------------------------------------------------------------- launch 3
// The 8-bit shared expert's gate/up rows i0 + lane/8 of this workgroup's block (planned
// expert d; every token chose it): lane takes groups lane%8, lane%8 + 8, ...; a group is 64
// code bytes per matrix, dotted with the tokens' staged x as exact bf16 code pairs.
__device__ __forceinline__ void batch_gate_up_q8_shared(const BatchParams& p, int rblk, int d) {
  extern __shared__ __align__(16) uint32_t smem[];
  const int H = p.L.hidden, I = p.L.inter, k = p.L.top_k, B = p.B;
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int CH = H >> 5, G = H >> 6;
  const int i0 = rblk * kGateUpRows + wv * 8;
  const int row = min(i0 + (lane >> 3), I - 1), gl = lane & 7;
  const uint4* gq = reinterpret_cast<const uint4*>(p.L.sh_gate.codes) + (int64_t)row * (H >> 4);
  const uint4* uq = reinterpret_cast<const uint4*>(p.L.sh_up.codes) + (int64_t)row * (H >> 4);
  const uint16_t* gs = p.L.sh_gate.scales + (int64_t)row * G;
  const uint16_t* gb = p.L.sh_gate.biases + (int64_t)row * G;
  const uint16_t* us = p.L.sh_up.scales + (int64_t)row * G;
  const uint16_t* ub = p.L.sh_up.biases + (int64_t)row * G;
  // stage x of every token (all chose the shared expert)
  constexpr int ST = chunk_stride<1>();
  uint32_t* vp = smem;
  float* vs = reinterpret_cast<float*>(vp + (size_t)B * CH * ST);
  for (int i = threadIdx.x; i < B * CH; i += blockDim.x) {
    const int b = i / CH, c = i - b * CH;
    stage_bf16_chunk(p.X + (size_t)b * H, c, vp + (size_t)i * ST, vs + i);
  }
  __syncthreads();
  float ag[kMaxBatch], au[kMaxBatch];
#pragma unroll
  for (int t = 0; t < kMaxBatch; ++t) ag[t] = au[t] = 0.f;
  for (int g = gl; g < G; g += 8) {
    uint4 cg[4], cu[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cg[q] = gq[4 * g + q];
      cu[q] = uq[4 * g + q];
    }
    const float sg = bf16_bits_to_f32(gs[g]), bg = bf16_bits_to_f32(gb[g]);
    const float su = bf16_bits_to_f32(us[g]), bu = bf16_bits_to_f32(ub[g]);
#pragma unroll
    for (int t = 0; t < kMaxBatch; ++t) {
      if (t >= B) break;
      const uint32_t* v = vp + ((size_t)t * CH + 2 * g) * ST;
      const float vsum = vs[t * CH + 2 * g] + vs[t * CH + 2 * g + 1];
      const float pg = q8_chunk_pdot<1>(cg[0], cg[1], v) + q8_chunk_pdot<1>(cg[2], cg[3], v + ST);
      const float pu = q8_chunk_pdot<1>(cu[0], cu[1], v) + q8_chunk_pdot<1>(cu[2], cu[3], v + ST);
      ag[t] += fmaf(sg, pg, bg * vsum);
      au[t] += fmaf(su, pu, bu * vsum);
    }
  }
  const int nslot = k + 1;
  const int i = i0 + (lane >> 3);
#pragma unroll
  for (int t = 0; t < kMaxBatch; ++t) {
    if (t >= B) break;
    const float g = group_sum_rt(ag[t], 3), u = group_sum_rt(au[t], 3);
    if ((lane & 7) == 0 && i < I) p.act[((size_t)t * nslot + k) * I + i] = silu(g) * u;
  }
  (void)d;
}

__global__ __launch_bounds__(kThreads) void batch_gate_up_kernel(BatchParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  const int H = p.L.hidden, I = p.L.inter, k = p.L.top_k, B = p.B;
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int per_expert = (I + kGateUpRows - 1) / kGateUpRows;
  const int d = blockIdx.x / per_expert, rblk = blockIdx.x - d * per_expert;
  const BatchPlan* plan = p.plan;
  if (d >= plan->n) return;  // beyond this step's experts (uniform)
  const int e = plan->expert[d];

  if (e < 0 && p.L.sh_q8) {  // the shared expert in 8-bit codes
    batch_gate_up_q8_shared(p, rblk, d);
    return;
  }
  // this lane's weights: row i0 + lane/8, groups lane%8 + 8q
  const Q4Mat& gm = e >= 0 ? p.L.gate : p.L.sh_gate;
  const Q4Mat& um = e >= 0 ? p.L.up : p.L.sh_up;
  const int CH = H >> 5, G = H >> 6;
  const int i0 = rblk * kGateUpRows + wv * 8;
  const int row = min(i0 + (lane >> 3), I - 1), gl = lane & 7;
  const int64_t oc = (e >= 0 ? e : 0) * (int64_t)I * (H >> 3), og = (e >= 0 ? e : 0) * (int64_t)I * G;
  const uint4* gc = reinterpret_cast<const uint4*>(gm.codes + oc) + (int64_t)row * CH;
  const uint4* uc = reinterpret_cast<const uint4*>(um.codes + oc) + (int64_t)row * CH;
  const uint16_t* gs = gm.scales + og + (int64_t)row * G;
  const uint16_t* gb = gm.biases + og + (int64_t)row * G;
  const uint16_t* us = um.scales + og + (int64_t)row * G;
  const uint16_t* ub = um.biases + og + (int64_t)row * G;
  constexpr int IT = 4;  // groups per lane per round (hidden 2048: one round)
  uint4 cg[IT][2], cu[IT][2];
  uint32_t sg[IT], bg[IT], su[IT], bu[IT];
  auto load = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int g = min(base + gl + 8 * q, G - 1);  // groups past the end: loaded, not used
      cg[q][0] = gc[2 * g];
      cg[q][1] = gc[2 * g + 1];
      cu[q][0] = uc[2 * g];
      cu[q][1] = uc[2 * g + 1];
      sg[q] = gs[g];
      bg[q] = gb[g];
      su[q] = us[g];
      bu[q] = ub[g];
    }
  };
  load(0);

  // the slots by which tokens 0..7 chose this expert (-1: not chosen), the same in every lane
  const uint2 sw = *reinterpret_cast<const uint2*>(&plan->slot[d][0]);
  auto slot_of = [&](int b) __attribute__((always_inline)) {
    return (int)(int8_t)(((b < 4 ? sw.x : sw.y) >> (8 * (b & 3))) & 0xFFu);
  };
  uint32_t chosen = 0;  // bit b: token b chose this expert
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) chosen |= (b < B && slot_of(b) >= 0 ? 1u : 0u) << b;

  // stage x of those tokens at their token index: [B] x [CH][ST1] pairs, then [B] x [CH] sums
  constexpr int ST = chunk_stride<1>();
  uint32_t* vp = smem;
  float* vs = reinterpret_cast<float*>(vp + (size_t)B * CH * ST);
  for (int i = threadIdx.x; i < B * CH; i += blockDim.x) {
    const int b = i / CH, c = i - b * CH;
    if (chosen >> b & 1u) stage_bf16_chunk(p.X + (size_t)b * H, c, vp + (size_t)i * ST, vs + i);
  }
  __syncthreads();

  float ag[kMaxBatch], au[kMaxBatch];
#pragma unroll
  for (int t = 0; t < kMaxBatch; ++t) ag[t] = au[t] = 0.f;
  for (int base = 0; base < G; base += 8 * IT) {  // wave-uniform trip count
    if (base > 0) load(base);
#pragma unroll
    for (int t = 0; t < kMaxBatch; ++t) {
      if (!(chosen >> t & 1u)) continue;
      const uint32_t* vt = vp + (size_t)t * CH * ST;
      const float* st = vs + t * CH;
#pragma unroll
      for (int q = 0; q < IT; ++q) {
        const int g = base + gl + 8 * q;
        const int gq = min(g, G - 1);
        const uint32_t* v = vt + 2 * gq * ST;
        const float vsum = st[2 * gq] + st[2 * gq + 1];
        const float tg = affine_term(chunk_pdot<1>(cg[q][0], v) + chunk_pdot<1>(cg[q][1], v + ST), vsum, sg[q], bg[q]);
        const float tu = affine_term(chunk_pdot<1>(cu[q][0], v) + chunk_pdot<1>(cu[q][1], v + ST), vsum, su[q], bu[q]);
        if (g < G) {
          ag[t] += tg;
          au[t] += tu;
        }
      }
    }
  }
  const int nslot = k + (p.L.has_shared ? 1 : 0);
  const int i = i0 + (lane >> 3);
#pragma unroll
  for (int t = 0; t < kMaxBatch; ++t) {
    if (!(chosen >> t & 1u)) continue;
    const float g = group_sum_rt(ag[t], 3), u = group_sum_rt(au[t], 3);
    if ((lane & 7) == 0 && i < I) p.act[((size_t)t * nslot + slot_of(t)) * I + i] = silu(g) * u;
  }
}

// ---------------------------------------------------------------- launch 4
__global__ __launch_bounds__(kThreads) void batch_down_kernel(BatchParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ float s_w[kMaxBatch][kMaxTopK + 1];
  __shared__ float s_red[kWaves][kMaxBatch][kDownRows];
  __shared__ int16_t s_list[kMaxPlan];
  __shared__ int s_nlist;

  const int H = p.L.hidden, I = p.L.inter, k = p.L.top_k;
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int b0 = blockIdx.y * p.tpp, nb = min(p.tpp, p.B - b0);
  const int n0 = blockIdx.x * kDownRows;
  const int nslot = k + (p.L.has_shared ? 1 : 0);
  const BatchPlan* plan = p.plan;
  const int nall = plan->n;
  // the planned experts chosen by a token of this pass, in plan order (wave 0, 64 entries per ballot)
  if (wv == 0) {
    int cnt = 0;
    for (int d0 = 0; d0 < nall; d0 += kWave) {
      const int dd = d0 + lane;
      const uint2 sw = dd < nall ? *reinterpret_cast<const uint2*>(&plan->slot[dd][0]) : make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
      bool mine = false;
#pragma unroll
      for (int b = 0; b < kMaxBatch; ++b) {
        const int j = (int)(int8_t)(((b < 4 ? sw.x : sw.y) >> (8 * (b & 3))) & 0xFFu);
        mine |= b >= b0 && b < b0 + nb && j >= 0;
      }
      const unsigned long long m = __ballot(mine);
      if (mine) s_list[cnt + __popcll(m & ((1ull << lane) - 1ull))] = (int16_t)dd;
      cnt += __popcll(m);
    }
    if (lane == 0) s_nlist = cnt;
  }
  __syncthreads();
  // an 8-bit shared expert (the plan's last entry, chosen by every token) is taken apart below
  const bool q8sh = p.L.has_shared && p.L.sh_q8;
  const int nplan = s_nlist - (q8sh ? 1 : 0);

  // lane: row n0 + lane / 8, groups sub, sub + 8, ...; wave w takes planned experts w, w + 4, ...
  const int sub = lane & (kDownLanes - 1), rsub = lane / kDownLanes;
  const int GI = I >> 6, CI = I >> 5;
  const int n = min(n0 + rsub, H - 1);
  const int64_t mat_codes = (int64_t)H * (I >> 3), mat_groups = (int64_t)H * GI;
  struct DownRow {
    uint4 c0, c1;
    uint32_t s, b;
  };
  auto load_row = [&](int li, int g) __attribute__((always_inline)) {
    DownRow r;
    const int e = plan->expert[s_list[li]];
    const Q4Mat& m = e >= 0 ? p.L.down : p.L.sh_down;
    const int64_t oc = e >= 0 ? e * mat_codes : 0, og = e >= 0 ? e * mat_groups : 0;
    const uint4* cr = reinterpret_cast<const uint4*>(m.codes + oc) + (int64_t)n * CI;
    const int gq = min(g, GI - 1);
    r.c0 = cr[2 * gq];
    r.c1 = cr[2 * gq + 1];
    r.s = m.scales[og + (int64_t)n * GI + gq];
    r.b = m.biases[og + (int64_t)n * GI + gq];
    return r;
  };
  // the first experts' rows are loaded before the staging below
  DownRow pf[kDownPrefetch];
  if (nplan > 0) {
#pragma unroll
    for (int q = 0; q < kDownPrefetch; ++q) pf[q] = load_row(min(wv + kWaves * q, nplan - 1), sub);
  }

  for (int i = threadIdx.x; i < nb * (k + 1); i += blockDim.x) {
    const int b = i / (k + 1), j = i - b * (k + 1);
    s_w[b][j] = p.wts[(b0 + b) * (k + 1) + j];  // slot k: the shared expert's weight
  }
  // stage the SwiGLU outputs of these tokens: [nb][nslot] x ([CI][ST2] pairs, [CI] sums)
  constexpr int ST = chunk_stride<2>();
  uint32_t* ap = smem;
  float* as = reinterpret_cast<float*>(ap + (size_t)p.tpp * nslot * CI * ST);
  for (int i = threadIdx.x; i < nb * nslot * CI; i += blockDim.x) {
    const int v = i / CI, c = i - v * CI;  // v = b * nslot + slot
    stage_f32_split_chunk(p.act + ((size_t)b0 * nslot + v) * I, c, ap + (size_t)i * ST, as + i);
  }
  __syncthreads();

  float acc[kMaxBatch];
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) acc[b] = 0.f;
  auto apply = [&](int li, int g, const DownRow& r) __attribute__((always_inline)) {
    const int dd = s_list[li];
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b >= nb) break;
      const int j = plan->slot[dd][b0 + b];
      if (j < 0) continue;
      const size_t vi = ((size_t)b * nslot + j) * CI + 2 * g;
      const uint32_t* v = ap + vi * ST;
      const float part = affine_term(chunk_pdot<2>(r.c0, v) + chunk_pdot<2>(r.c1, v + ST), as[vi] + as[vi + 1], r.s, r.b);
      acc[b] = fmaf(s_w[b][j], part, acc[b]);
    }
  };
  for (int q0 = 0; wv + kWaves * q0 < nplan; q0 += kDownPrefetch) {
    if (q0 > 0) {
#pragma unroll
      for (int q = 0; q < kDownPrefetch; ++q) pf[q] = load_row(min(wv + kWaves * (q0 + q), nplan - 1), sub);
    }
#pragma unroll
    for (int q = 0; q < kDownPrefetch; ++q) {
      const int dd = wv + kWaves * (q0 + q);
      if (dd < nplan && sub < GI) apply(dd, sub, pf[q]);
    }
    if (GI > kDownLanes) {  // rows longer than 8 groups: the further groups, loaded as they are used
      for (int q = 0; q < kDownPrefetch; ++q) {
        const int dd = wv + kWaves * (q0 + q);
        if (dd >= nplan) break;
        for (int g = sub + kDownLanes; g < GI; g += kDownLanes) apply(dd, g, load_row(dd, g));
      }
    }
  }
  if (q8sh && wv == nplan % kWaves) {
    // 8-bit shared down row n: group g is 64 code bytes, chunks 2g and 2g + 1 of slot k
    const uint4* cr = reinterpret_cast<const uint4*>(p.L.sh_down.codes) + (int64_t)n * (I >> 4);
    const uint16_t* sr = p.L.sh_down.scales + (int64_t)n * GI;
    const uint16_t* br = p.L.sh_down.biases + (int64_t)n * GI;
    for (int g = sub; g < GI; g += kDownLanes) {
      const uint4 c0 = cr[4 * g], c1 = cr[4 * g + 1], c2 = cr[4 * g + 2], c3 = cr[4 * g + 3];
      const float sc = bf16_bits_to_f32(sr[g]), bi = bf16_bits_to_f32(br[g]);
#pragma unroll
      for (int b = 0; b < kMaxBatch; ++b) {
        if (b >= nb) break;
        const size_t vi = ((size_t)b * nslot + k) * CI + 2 * g;
        const uint32_t* v = ap + vi * ST;
        const float part = fmaf(sc, q8_chunk_pdot<2>(c0, c1, v) + q8_chunk_pdot<2>(c2, c3, v + ST),
                                bi * (as[vi] + as[vi + 1]));
        acc[b] = fmaf(s_w[b][k], part, acc[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) {
    if (b >= nb) break;
    const float r = group_sum_rt(acc[b], 3);
    if (sub == 0) s_red[wv][b][rsub] = r;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb * kDownRows; i += blockDim.x) {
    const int b = i / kDownRows, r = i - b * kDownRows, nn = n0 + r;
    if (nn >= H) continue;
    float t = s_red[0][b][r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += s_red[w][b][r];
    const size_t o = (size_t)(b0 + b) * H + nn;
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.y)[o] = (uint16_t)f32_to_bf16_bits(t);
    else
      reinterpret_cast<float*>(p.y)[o] = t;
  }
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t gate_up_lds(const DecodeLayer& L, int B) {
  return (size_t)B * (L.hidden >> 5) * (chunk_stride<1>() * 4 + 4);
}

size_t down_lds_per_token(const DecodeLayer& L) {
  const int nslot = L.top_k + (L.has_shared ? 1 : 0);
  return (size_t)nslot * (L.inter >> 5) * (chunk_stride<2>() * 4 + 4);
}

template <int NB>
void launch_route_plan(const BatchParams& p, int grid, hipStream_t stream) {
  if (p.L.router_q8.codes)
    hipLaunchKernelGGL((batch_route_kernel<NB, true>), dim3(grid), dim3(kRouteWaves * kWave), 0, stream, p);
  else
    hipLaunchKernelGGL((batch_route_kernel<NB, false>), dim3(grid), dim3(kRouteWaves * kWave), 0, stream, p);
  const dim3 one(1), threads(kRouteWaves * kWave);
  if (p.L.n_experts <= 4 * kWave)
    hipLaunchKernelGGL((batch_plan_kernel<NB, 4>), one, threads, 0, stream, p);
  else if (p.L.n_experts <= 8 * kWave)
    hipLaunchKernelGGL((batch_plan_kernel<NB, 8>), one, threads, 0, stream, p);
  else
    hipLaunchKernelGGL((batch_plan_kernel<NB, kMaxExperts / kWave>), one, threads, 0, stream, p);
}

}  // namespace

size_t decode_batch_workspace_bytes(int n_experts, int top_k, int inter, int B) {
  return align256((size_t)B * n_experts * 4) + align256(sizeof(BatchPlan)) + align256((size_t)B * (top_k + 1) * 4) +
         align256((size_t)B * (top_k + 1) * inter * 4);
}

bool decode_batch_supported(const DecodeLayer& L, int B, size_t max_lds) {
  // the down launch needs room for at least one token's SwiGLU outputs
  return gate_up_lds(L, B) <= max_lds && down_lds_per_token(L) <= max_lds;
}

hipError_t run_moe_ffn_decode_batch(const DecodeLayer& L, const uint16_t* X, int B, void* y, int out_bf16,
                                    int32_t* ids_out, float* w_out, void* ws, size_t max_lds, hipStream_t stream) {
  BatchParams p{};
  p.L = L;
  p.X = X;
  p.B = B;
  char* w = static_cast<char*>(ws);
  p.logits = reinterpret_cast<float*>(w);
  w += align256((size_t)B * L.n_experts * 4);
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
  p.tpp = (int)std::min<size_t>((size_t)B, max_lds / per_tok);

  const int rgrid = (L.n_experts + kRouteWaves - 1) / kRouteWaves;
  switch (B) {
    case 1: launch_route_plan<1>(p, rgrid, stream); break;
    case 2: launch_route_plan<2>(p, rgrid, stream); break;
    case 3: launch_route_plan<3>(p, rgrid, stream); break;
    case 4: launch_route_plan<4>(p, rgrid, stream); break;
    case 5: launch_route_plan<5>(p, rgrid, stream); break;
    case 6: launch_route_plan<6>(p, rgrid, stream); break;
    case 7: launch_route_plan<7>(p, rgrid, stream); break;
    default: launch_route_plan<8>(p, rgrid, stream); break;
  }
  const int nd_max = std::min(B * L.top_k, L.n_experts) + (L.has_shared ? 1 : 0);
  const int per_expert = (L.inter + kGateUpRows - 1) / kGateUpRows;
  hipLaunchKernelGGL(batch_gate_up_kernel, dim3(nd_max * per_expert), dim3(kThreads), gate_up_lds(L, B), stream, p);
  const int passes = (B + p.tpp - 1) / p.tpp;
  hipLaunchKernelGGL(batch_down_kernel, dim3((L.hidden + kDownRows - 1) / kDownRows, passes), dim3(kThreads),
                     (size_t)p.tpp * per_tok, stream, p);
  return hipGetLastError();
}

}  // namespace q4moe
