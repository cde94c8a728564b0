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
// No grid-wide barrier: every value handed from one workgroup to another (the
// router logits, the SwiGLU activations) is published as one 64-bit word
// {epoch, fp32 bits} of this launch, so a consumer's load both reads the value
// and tells whether it is there yet; only late words are polled again.  The
// activations are produced 8 rows at a time, and the 8 words of a 64-byte line
// are written by one store instruction of one wave.  The epoch is agreed through
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
constexpr unsigned kPollLimit = 1u << 18;  // ~0.25 s of polling

constexpr int kMaxBlocks = 1024;

struct DecodeWs {
  unsigned long long group_ctr[kEpochGroups][32];  // {epoch:hi32, arrivals:lo32}, one 256-byte slot each
  unsigned timeouts;
  unsigned pad[63];
  // Router logit of expert e: tag_logit[e] = {epoch:hi32, fp32 bits:lo32}.  The
  // 8 words of a 64-byte line are written by one store instruction of one wave
  // (lines shared by several writers slow their observers down severalfold).
  unsigned long long tag_logit[kMaxExperts];
};

struct DecodeParams {
  const uint16_t* x;          // [H]
  void* y;                    // [H]
  int out_mode;               // kOutF32, kOutBf16, kOutBf16Residual
  int32_t* ids_out;           // nullable [k]
  float* w_out;               // nullable [k]
  DecodeWs* ws;
  unsigned long long* act;    // [k+1][I] tagged SwiGLU outputs: routed slots 0..k-1, shared slot k
  int lsH;                    // log2 lanes per row for rows of length hidden
  int lsI;                    // log2 lanes per row for rows of length inter
  DecodeLayer L;              // last: the per-call fields above keep fixed small offsets
};

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

// Padded row length (floats) of a 64-column group in the fp32 LDS copies that an
// 8-bit shared expert is read against (the padding puts the groups of neighbouring
// lanes on different banks).
constexpr int kQ8Pad = 68;

// Stage `nvec` tagged fp32 vectors of n values each (contiguous, published by
// other workgroups as {epoch, bits} words; nvec * n a multiple of 32) as hi/lo
// bf16 parts.  Lane-contiguous 16-byte device-coherent loads (two words per
// lane, all rounds in flight together); only pairs not yet complete are loaded
// again (bounded; a timeout is counted).  A lane quad holds one 8-value block:
// lanes 0-1 of the quad assemble its permuted pair words from their own values
// and the matching ones of lanes 2-3; 16 lanes hold one 32-value chunk.  With f32_dst, the
// values from flat index f32_first on are also written as fp32 in kQ8Pad-padded groups.
constexpr int kTagRounds = 9;  // 16-byte loads per thread: 9 x 256 x 2 words = 4608 = 9 slots x 512

__device__ __forceinline__ void stage_tagged_split(const unsigned long long* src, int nvec, int n, uint32_t* vp,
                                                   float* vs, uint32_t epoch, unsigned* timeouts,
                                                   float* f32_dst = nullptr, int f32_first = 0) {
  constexpr int ST = chunk_stride<2>();
  const int t = threadIdx.x, nthr = blockDim.x;
  const int npairs = (nvec * n) >> 1;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned long long*>(src), 0, npairs * 16, kBufferRsrcWord3);
  for (int base = 0; base < npairs; base += nthr * kTagRounds) {
    uint4 w[kTagRounds];
    auto fetch = [&](int r) __attribute__((always_inline)) {
      const int q = base + r * nthr + t;  // past the end: the bounds check returns zeros, not used
      w[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, q * 16, 0, kLoadDeviceScope));
    };
    auto complete = [&](int r) __attribute__((always_inline)) { return w[r].y == epoch && w[r].w == epoch; };
#pragma unroll
    for (int r = 0; r < kTagRounds; ++r) fetch(r);
#pragma unroll
    for (int r = 0; r < kTagRounds; ++r) {
      if (base + r * nthr + t >= npairs) continue;
      for (unsigned spins = 0; !complete(r); ++spins) {
        if (spins == kPollLimit) {
          __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        fetch(r);
      }
    }
#pragma unroll
    for (int r = 0; r < kTagRounds; ++r) {
      const int q = base + r * nthr + t;
      const bool ok = q < npairs;
      // this lane's values j0, j0 + 1 of block q / 4, j0 = 2 * (q % 4)
      const float v0 = ok ? __uint_as_float(w[r].x) : 0.f, v1 = ok ? __uint_as_float(w[r].z) : 0.f;
      const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
      const uint32_t l0 = f32_to_bf16_bits(v0 - bf16_bits_to_f32(h0)), l1 = f32_to_bf16_bits(v1 - bf16_bits_to_f32(h1));
      const float part = (bf16_bits_to_f32(h0) + bf16_bits_to_f32(l0)) + (bf16_bits_to_f32(h1) + bf16_bits_to_f32(l1));
      if (f32_dst && ok && 2 * q >= f32_first) {  // values from f32_first on, also as fp32 in padded groups
        const int i = 2 * q - f32_first;
        *reinterpret_cast<float2*>(f32_dst + (i >> 6) * kQ8Pad + (i & 63)) = make_float2(v0, v1);
      }
      // values j0 + 4, j0 + 5 from the lane two places over in the quad
      const uint32_t hh = dpp_u32<kDppQuadXor2>(h0 | h1 << 16), ll = dpp_u32<kDppQuadXor2>(l0 | l1 << 16);
      if (ok && (q & 2) == 0) {
        const int b = q >> 2, j0 = 2 * (q & 3);
        uint32_t* dst = vp + (b >> 2) * ST + (b & 3) * 4 + j0;
        *reinterpret_cast<uint2*>(dst) = make_uint2(h0 | (hh & 0xFFFFu) << 16, h1 | (hh >> 16) << 16);
        *reinterpret_cast<uint2*>(dst + 16) = make_uint2(l0 | (ll & 0xFFFFu) << 16, l1 | (ll >> 16) << 16);
      }
      const float sum = group_sum_rt(part, 4);
      if (ok && (q & 15) == 0) vs[q >> 4] = sum;
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

// Gate/up of rows i0..i0+7 of one expert (e >= 0: routed expert e; e < 0: the
// shared expert) over groups [g_lo, g_hi) against the staged x: lane l takes
// row i0 + l/8 and groups g_lo + l%8 + 8t, with IT groups' loads in flight per
// lane; every lane of a row's 8-lane group returns that row's partial (g, u).
// Rows past I are read clamped and their results are not used.
constexpr int kUnitRows = 8;

template <int IT>
__device__ __forceinline__ float2 unit_gate_up(const DecodeLayer& L, int e, int i0, int g_lo, int g_hi,
                                               const uint32_t* vp, const float* vs) {
  constexpr int ST = chunk_stride<1>();
  const int H = L.hidden, I = L.inter;
  const int lane = lane_id();
  const int row = min(i0 + (lane >> 3), I - 1), gl = lane & 7;
  const GateUpRef ref =
      e >= 0 ? gate_up_ref(L.gate, L.up, e, row, H, I) : gate_up_ref(L.sh_gate, L.sh_up, 0, row, H, I);
  float ag = 0.f, au = 0.f;
  for (int base = g_lo; base < g_hi; base += 8 * IT) {  // wave-uniform trip count
    uint4 gc[IT][2], uc[IT][2];
    uint32_t gs[IT], gb[IT], us[IT], ub[IT];
#pragma unroll
    for (int t = 0; t < IT; ++t) {
      const int g = min(base + gl + 8 * t, g_hi - 1);  // groups past the range: loaded, not used
      gc[t][0] = ref.gc[2 * g];
      gc[t][1] = ref.gc[2 * g + 1];
      uc[t][0] = ref.uc[2 * g];
      uc[t][1] = ref.uc[2 * g + 1];
      gs[t] = ref.gs[g];
      gb[t] = ref.gb[g];
      us[t] = ref.us[g];
      ub[t] = ref.ub[g];
    }
#pragma unroll
    for (int t = 0; t < IT; ++t) {
      const int g = base + gl + 8 * t;
      const int gc_ = min(g, g_hi - 1);
      const uint32_t* v = vp + 2 * gc_ * ST;
      const float vsum = vs[2 * gc_] + vs[2 * gc_ + 1];
      const float tg = affine_term(chunk_pdot<1>(gc[t][0], v) + chunk_pdot<1>(gc[t][1], v + ST), vsum, gs[t], gb[t]);
      const float tu = affine_term(chunk_pdot<1>(uc[t][0], v) + chunk_pdot<1>(uc[t][1], v + ST), vsum, us[t], ub[t]);
      if (g < g_hi) {
        ag += tg;
        au += tu;
      }
    }
  }
  return make_float2(group_sum_rt(ag, 3), group_sum_rt(au, 3));
}

// An 8-bit shared expert (affine Q8, code j of a row in byte j % 4 of word j / 4)
// is read against fp32 copies of its input in LDS, one 64-column group per row of
// kQ8Pad floats: the 64 values, then (for x) their sum.  Its gate/up units are 8 rows
// of 8 lanes, as for 4-bit codes.
constexpr int kQ8UnitRows = 8, kQ8LaneLog = 3;

// Stage a vector of n values (n a multiple of 64; value i from get(i)) into padded
// groups with their sums, one group per wave at a time.
template <class Get>
__device__ __forceinline__ void stage_q8_groups(float* dst, int n, Get get) {
  const int lane = lane_id();
  for (int g = threadIdx.x / kWave; g < (n >> 6); g += kThreads / kWave) {
    const float v = get(g * 64 + lane);
    dst[g * kQ8Pad + lane] = v;
    const float t = group_sum_rt(v, 6);
    if (lane == 0) dst[g * kQ8Pad + 64] = t;
  }
}

// scale * sum(q v) + bias * sum(v) over one 64-column group of an 8-bit row, for
// two rows (a: codes ca, b: codes cb) against the same 64 values v.
__device__ __forceinline__ float2 q8_group_terms2(const uint4* ca, const uint4* cb, const float* v, uint32_t sa,
                                                  uint32_t ba, uint32_t sb, uint32_t bb) {
  uint4 wa[4], wb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    wa[q] = ca[q];
    wb[q] = cb[q];
  }
  float pa = 0.f, pb = 0.f;
  const float sv = v[64];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a[4] = {wa[q].x, wa[q].y, wa[q].z, wa[q].w}, b[4] = {wb[q].x, wb[q].y, wb[q].z, wb[q].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(v + 16 * q + 4 * w);
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pa = fmaf(xv[i], (float)((a[w] >> (8 * i)) & 0xFFu), pa);
        pb = fmaf(xv[i], (float)((b[w] >> (8 * i)) & 0xFFu), pb);
      }
    }
  }
  return make_float2(fmaf(bf16_bits_to_f32(sa), pa, bf16_bits_to_f32(ba) * sv),
                     fmaf(bf16_bits_to_f32(sb), pb, bf16_bits_to_f32(bb) * sv));
}

// The same for one row whose 64 codes are already in registers.
__device__ __forceinline__ float q8_group_term_regs(const uint4 (&w4)[4], const float* v, uint32_t s, uint32_t b) {
  float p = 0.f, sv = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a[4] = {w4[q].x, w4[q].y, w4[q].z, w4[q].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(v + 16 * q + 4 * w);
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv += xv[i];
        p = fmaf(xv[i], (float)((a[w] >> (8 * i)) & 0xFFu), p);
      }
    }
  }
  return fmaf(bf16_bits_to_f32(s), p, bf16_bits_to_f32(b) * sv);
}

// The same for one row read from memory.
__device__ __forceinline__ float q8_group_term(const uint4* c, const float* v, uint32_t s, uint32_t b) {
  uint4 w4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) w4[q] = c[q];
  return q8_group_term_regs(w4, v, s, b);
}

// Gate/up of rows i0..i0+3 of an 8-bit shared expert over groups [g_lo, g_hi): lane l
// takes row i0 + l/16 and groups g_lo + l%16 + 16t, two groups' loads in flight; every
// lane of a row's 16-lane group returns that row's (g, u).  xf is the input in padded groups.
__device__ __forceinline__ float2 unit_gate_up_q8(const DecodeLayer& L, int i0, int g_lo, int g_hi, const float* xf) {
  constexpr int LPR = 1 << kQ8LaneLog;
  const int H = L.hidden, I = L.inter, G = H >> 6;
  const int lane = lane_id();
  const int row = min(i0 + (lane >> kQ8LaneLog), I - 1), gl = lane & (LPR - 1);
  const uint4* gc = reinterpret_cast<const uint4*>(L.sh_gate.codes) + (int64_t)row * (H >> 4);
  const uint4* uc = reinterpret_cast<const uint4*>(L.sh_up.codes) + (int64_t)row * (H >> 4);
  const uint16_t* gs = L.sh_gate.scales + (int64_t)row * G;
  const uint16_t* gb = L.sh_gate.biases + (int64_t)row * G;
  const uint16_t* us = L.sh_up.scales + (int64_t)row * G;
  const uint16_t* ub = L.sh_up.biases + (int64_t)row * G;
  float ag = 0.f, au = 0.f;
  for (int base = g_lo; base < g_hi; base += 2 * LPR) {  // wave-uniform trip count
    // groups past the range are read clamped (in bounds) and their terms dropped
    const bool ok0 = base + gl < g_hi, ok1 = base + gl + LPR < g_hi;
    const int g0 = min(base + gl, g_hi - 1), g1 = min(base + gl + LPR, g_hi - 1);
    const float2 t0 = q8_group_terms2(gc + 4 * g0, uc + 4 * g0, xf + g0 * kQ8Pad, gs[g0], gb[g0], us[g0], ub[g0]);
    const float2 t1 = q8_group_terms2(gc + 4 * g1, uc + 4 * g1, xf + g1 * kQ8Pad, gs[g1], gb[g1], us[g1], ub[g1]);
    if (ok0) {
      ag += t0.x;
      au += t0.y;
    }
    if (ok1) {
      ag += t1.x;
      au += t1.y;
    }
  }
  return make_float2(group_sum_rt(ag, kQ8LaneLog), group_sum_rt(au, kQ8LaneLog));
}

// Gate/up of a shared-expert unit in the shared expert's format.
template <bool kQ8Shared, int IT>
__device__ __forceinline__ float2 shared_unit_gate_up(const DecodeLayer& L, int i0, int g_lo, int g_hi,
                                                      const uint32_t* vp, const float* vs, const float* xf) {
  if constexpr (kQ8Shared)
    return unit_gate_up_q8(L, i0, g_lo, g_hi, xf);
  else
    return unit_gate_up<IT>(L, -1, i0, g_lo, g_hi, vp, vs);
}

// Publish the SwiGLU outputs of a unit's rows as tagged words: the 8 lanes that
// hold rows i0..i0+7 (lane % 8 == 0) write one 64-byte line together.
template <int LOG = 3>
__device__ __forceinline__ void publish_unit(unsigned long long* act_slot, int i0, int I, float a, uint32_t epoch) {
  const int lane = lane_id();
  const int i = i0 + (lane >> LOG);
  if ((lane & ((1 << LOG) - 1)) == 0 && i < I)
    __hip_atomic_store(act_slot + i, ((unsigned long long)epoch << 32) | __float_as_uint(a), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
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
__device__ __forceinline__ void wave_topk_tagged(const unsigned long long* tags, int E, int k, uint32_t epoch,
                                                 unsigned* timeouts, int32_t* s_ids, float* s_w, int32_t* ids_out,
                                                 float* w_out) {
  static_assert(V % 2 == 0, "two tagged words per 16-byte load");
  const int lane = lane_id();
  uint32_t key[V];
  int id[V];
#pragma unroll
  for (int j = 0; j < V; ++j) id[j] = lane * V + j;
  // lane-contiguous 16-byte device-coherent loads; words past E read as zeros (bounds check)
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned long long*>(tags), 0, E * 8, kBufferRsrcWord3);
  for (unsigned spins = 0;; ++spins) {
    bool ready = true;
    uint4 t[V / 2];
#pragma unroll
    for (int h = 0; h < V / 2; ++h)  // all loads in flight together
      t[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (lane * V + 2 * h) * 8, 0,
                                                                          kLoadDeviceScope));
#pragma unroll
    for (int h = 0; h < V / 2; ++h) {
      key[2 * h] = t[h].x;
      key[2 * h + 1] = t[h].z;
      ready &= id[2 * h] >= E || t[h].y == epoch;
      ready &= id[2 * h + 1] >= E || t[h].w == epoch;
    }
    if (__all(ready)) break;
    if (spins == kPollLimit) {
      if (lane == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int j = 0; j < V; ++j) key[j] = id[j] < E ? float_key(__uint_as_float(key[j])) : 0u;
  wave_topk_keys<V>(key, id, k, s_ids, s_w);
  if (lane < k) {
    if (ids_out) ids_out[lane] = s_ids[lane];
    if (w_out) w_out[lane] = s_w[lane];
  }
}

// The shared-expert unit of workgroup b when each workgroup takes at most one
// (units + router workgroups <= grid): the workgroups after the router ones, so
// no workgroup computes both; -1 for none.
__device__ __forceinline__ int shared_unit_of(int b, int grid, int rgroups, int units) {
  const int su = b - rgroups;
  return units + rgroups <= grid && su >= 0 && su < units ? su : -1;
}

struct DownPrefetch {
  uint4 c0, c1;
  uint32_t s, b;
};

// The layer's body, specialised on the router's format (bf16, or 8-bit affine codes) and on
// a shared-expert gate (the shared expert weighted by sigmoid(sh_gate_w . x)) and on
// the shared expert's code width (4 or 8 bits).
template <bool kQ8Router, bool kShGate, bool kQ8Shared>
__device__ __forceinline__ void decode_layer(DecodeParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ int32_t s_ids[kMaxTopK + 1];
  __shared__ float s_w[kMaxTopK + 1];
  __shared__ float s_red[kWaves][kWave];
  __shared__ float2 s_pair[kWaves / 2][kUnitRows];
  __shared__ float2 s_third[kWaves - 1][kUnitRows];
  __shared__ float s_rlog[2 * kWaves];
  __shared__ uint32_t s_epoch;

  const int H = p.L.hidden, I = p.L.inter, E = p.L.n_experts, k = p.L.top_k;
  const int CH = H >> 5, CI = I >> 5;
  const int nslot = k + (p.L.has_shared ? 1 : 0);
  uint32_t* xp = smem;                                                                // [CH][ST1]
  float* xs = reinterpret_cast<float*>(xp + CH * chunk_stride<1>());                   // [CH]
  uint32_t* ap = reinterpret_cast<uint32_t*>(xs + CH);                                // [nslot][CI][ST2]
  float* as = reinterpret_cast<float*>(ap + (size_t)nslot * CI * chunk_stride<2>());  // [nslot][CI]
  const size_t xf_off = (reinterpret_cast<const uint32_t*>(as + (size_t)nslot * CI) - smem + 3) & ~size_t(3);
  float* xf = reinterpret_cast<float*>(smem + xf_off);
  // (xf: 8-bit shared expert only, x as fp32 [H/64][kQ8Pad], 16-byte aligned)
  float* af = xf + (size_t)(H >> 6) * kQ8Pad;         // 8-bit shared expert: its activations [I/64][kQ8Pad]
  unsigned* timeouts = &p.ws->timeouts;

  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;

  // ---- epoch of this launch: the arrivals of one group agree on its counter's
  // epoch field.  Taken by thread 0 once its first router loads are in flight,
  // so the two latencies overlap.
  auto acquire_epoch = [&]() {
    const int g = blockIdx.x % kEpochGroups;
    const unsigned gsize = (gridDim.x - g + kEpochGroups - 1) / kEpochGroups;
    unsigned long long* ctr = &p.ws->group_ctr[g][0];
    const unsigned long long old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)old == gsize - 1)
      __hip_atomic_fetch_add(ctr, (1ull << 32) - gsize, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_epoch = (uint32_t)(old >> 32) + 1u;
  };

  // ------------------------------------------------------------ phase A
  // Router: workgroup b computes experts 8b..8b+7 (two per wave, x read from
  // global memory) and wave 0 publishes them as one line of tagged words.
  const int rgroups = (E + 7) / 8;
  bool have_epoch = false;
  constexpr bool router_q8 = kQ8Router;
  for (int rb = blockIdx.x; rb < rgroups; rb += gridDim.x) {  // same trip count for the whole workgroup
    const uint4* xv = reinterpret_cast<const uint4*>(p.x);
    float la, lb;
    if constexpr (router_q8) {
      // 8-bit router (count 1, [E][H/4] words): a lane takes 16-code chunks (one
      // 16-byte load per row), which lie inside one 64-column group, and adds
      // scale * sum(x q) + bias * sum(x) for each; x as 8 bf16 per 16-byte load.
      const int G = H >> 6;
      const int e0 = min(rb * 8 + 2 * wv, E - 1), e1 = min(rb * 8 + 2 * wv + 1, E - 1);
      const uint4* q0 = reinterpret_cast<const uint4*>(p.L.router_q8.codes) + (size_t)e0 * (H >> 4);
      const uint4* q1 = reinterpret_cast<const uint4*>(p.L.router_q8.codes) + (size_t)e1 * (H >> 4);
      float a = 0.f, b = 0.f;
      for (int c = lane; c < (H >> 4); c += kWave) {
        const uint4 w0 = q0[c], w1 = q1[c], xa = xv[2 * c], xb = xv[2 * c + 1];
        const int g = c >> 2;
        const float s0 = bf16_bits_to_f32(p.L.router_q8.scales[(size_t)e0 * G + g]);
        const float o0 = bf16_bits_to_f32(p.L.router_q8.biases[(size_t)e0 * G + g]);
        const float s1 = bf16_bits_to_f32(p.L.router_q8.scales[(size_t)e1 * G + g]);
        const float o1 = bf16_bits_to_f32(p.L.router_q8.biases[(size_t)e1 * G + g]);
        if (!have_epoch) {
          have_epoch = true;
          if (threadIdx.x == 0) acquire_epoch();
        }
        const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        const uint32_t c0w[4] = {w0.x, w0.y, w0.z, w0.w}, c1w[4] = {w1.x, w1.y, w1.z, w1.w};
        float p0 = 0.f, p1 = 0.f, xs_ = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float xi = bf16_bits_to_f32((xw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
          xs_ += xi;
          p0 = fmaf(xi, (float)((c0w[i >> 2] >> (8 * (i & 3))) & 0xFFu), p0);
          p1 = fmaf(xi, (float)((c1w[i >> 2] >> (8 * (i & 3))) & 0xFFu), p1);
        }
        a += fmaf(s0, p0, o0 * xs_);
        b += fmaf(s1, p1, o1 * xs_);
      }
      if (!have_epoch) {
        have_epoch = true;
        if (threadIdx.x == 0) acquire_epoch();
      }
      la = group_sum_rt(a, 6);
      lb = group_sum_rt(b, 6);
    } else {
    const uint4* r0 = reinterpret_cast<const uint4*>(p.L.router + (size_t)min(rb * 8 + 2 * wv, E - 1) * H);
    const uint4* r1 = reinterpret_cast<const uint4*>(p.L.router + (size_t)min(rb * 8 + 2 * wv + 1, E - 1) * H);
    constexpr int kBatch = 4;  // row chunks in flight per lane and row
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
    for (int c0 = 0; c0 < (H >> 3); c0 += kBatch * kWave) {
      uint4 w0[kBatch], w1[kBatch], v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int c = c0 + q * kWave + lane;
        const bool ok = c < (H >> 3);
        w0[q] = ok ? r0[c] : make_uint4(0, 0, 0, 0);
        w1[q] = ok ? r1[c] : make_uint4(0, 0, 0, 0);
        v[q] = ok ? xv[c] : make_uint4(0, 0, 0, 0);
      }
      if (!have_epoch) {
        have_epoch = true;
        if (threadIdx.x == 0) acquire_epoch();
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        a0 = dot2_bf16(w0[q].x, v[q].x, a0);
        a1 = dot2_bf16(w0[q].y, v[q].y, a1);
        a0 = dot2_bf16(w0[q].z, v[q].z, a0);
        a1 = dot2_bf16(w0[q].w, v[q].w, a1);
        b0 = dot2_bf16(w1[q].x, v[q].x, b0);
        b1 = dot2_bf16(w1[q].y, v[q].y, b1);
        b0 = dot2_bf16(w1[q].z, v[q].z, b0);
        b1 = dot2_bf16(w1[q].w, v[q].w, b1);
      }
    }
    la = group_sum_rt(a0 + a1, 6);
    lb = group_sum_rt(b0 + b1, 6);
    }
    if (lane == 0) {
      s_rlog[2 * wv] = la;
      s_rlog[2 * wv + 1] = lb;
    }
    __syncthreads();
    if (wv == 0 && lane < 8 && rb * 8 + lane < E)
      __hip_atomic_store(&p.ws->tag_logit[rb * 8 + lane], ((unsigned long long)s_epoch << 32) | __float_as_uint(s_rlog[lane]),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();  // s_rlog is reused
  }
  if (!have_epoch && threadIdx.x == 0) acquire_epoch();
  stage_bf16_parallel(p.x, H, xp, xs, 0, kThreads);
  if constexpr (kQ8Shared) stage_q8_groups(xf, H, [&](int i) { return bf16_bits_to_f32(p.x[i]); });
  __syncthreads();
  const uint32_t epoch = s_epoch;

  if (wv == 0) {
    // The shared expert's gate, sigmoid(sh_gate_w . x), taken while the router logits of the
    // other workgroups are still arriving (the top-k below waits for them).
    float sh_weight = 1.0f;
    if constexpr (kShGate) {
      const uint4* gw = reinterpret_cast<const uint4*>(p.L.sh_gate_w);
      const uint4* gx = reinterpret_cast<const uint4*>(p.x);
      float d0 = 0.f, d1 = 0.f;
      for (int c = lane; c < (H >> 3); c += kWave) {
        const uint4 a = gw[c], b = gx[c];
        d0 = dot2_bf16(a.x, b.x, d0);
        d1 = dot2_bf16(a.y, b.y, d1);
        d0 = dot2_bf16(a.z, b.z, d0);
        d1 = dot2_bf16(a.w, b.w, d1);
      }
      const float d = group_sum_rt(d0 + d1, 6);
      sh_weight = 1.0f / (1.0f + __expf(-d));
    }
    // B: top-k from the tagged logits (every workgroup, redundantly)
    if (E <= 4 * kWave)
      wave_topk_tagged<4>(p.ws->tag_logit, E, k, epoch, timeouts, s_ids, s_w, blockIdx.x == 0 ? p.ids_out : nullptr,
                          blockIdx.x == 0 ? p.w_out : nullptr);
    else
      wave_topk_tagged<kMaxExperts / kWave>(p.ws->tag_logit, E, k, epoch, timeouts, s_ids, s_w,
                                            blockIdx.x == 0 ? p.ids_out : nullptr, blockIdx.x == 0 ? p.w_out : nullptr);
    if (lane == 0 && p.L.has_shared) {
      s_ids[k] = -1;
      s_w[k] = sh_weight;
    }
  } else if (p.L.has_shared) {
    // A, off the critical path: the shared expert's gate/up in 8-row units.  With
    // at most one unit per workgroup, waves 1-3 split its groups in thirds and
    // wave 1 adds the thirds after the barrier below; otherwise each wave takes
    // whole units.
    constexpr int R = kQ8Shared ? kQ8UnitRows : kUnitRows, LOG = kQ8Shared ? kQ8LaneLog : 3;
    const int units = (I + R - 1) / R, G = H >> 6;
    const int su = shared_unit_of(blockIdx.x, gridDim.x, rgroups, units);
    if (units + rgroups <= (int)gridDim.x) {
      if (su >= 0) {
        const int w = wv - 1;
        const float2 gu = shared_unit_gate_up<kQ8Shared, 2>(p.L, su * R, w * G / 3, (w + 1) * G / 3, xp, xs, xf);
        if ((lane & ((1 << LOG) - 1)) == 0) s_third[w][lane >> LOG] = gu;
      }
    } else {
      for (int u = (wv - 1) * gridDim.x + blockIdx.x; u < units; u += (kWaves - 1) * gridDim.x) {
        const float2 gu = shared_unit_gate_up<kQ8Shared, 4>(p.L, u * R, 0, G, xp, xs, xf);
        publish_unit<LOG>(p.act + (size_t)k * I, u * R, I, silu(gu.x) * gu.y, epoch);
      }
    }
  }
  __syncthreads();
  if (p.L.has_shared && wv == 1) {
    constexpr int R = kQ8Shared ? kQ8UnitRows : kUnitRows, LOG = kQ8Shared ? kQ8LaneLog : 3;
    const int units = (I + R - 1) / R;
    const int su = shared_unit_of(blockIdx.x, gridDim.x, rgroups, units);
    if (units + rgroups <= (int)gridDim.x && su >= 0) {
      const float2 a = s_third[0][lane >> LOG], b = s_third[1][lane >> LOG], c = s_third[2][lane >> LOG];
      const float g = (a.x + b.x) + c.x, up = (a.y + b.y) + c.y;
      publish_unit<LOG>(p.act + (size_t)k * I, su * R, I, silu(g) * up, epoch);
    }
  }

  {
    // B: the routed experts' gate/up in 8-row units; the two waves of a pair
    // split the groups, one wave adds the halves and publishes the line.
    const int per_slot = (I + kUnitRows - 1) / kUnitRows;
    const int units = k * per_slot;
    const int pair = wv >> 1, half = wv & 1;
    const int G = H >> 6, gmid = (G + 1) >> 1;
    for (int ub = 2 * blockIdx.x; ub < units; ub += 2 * gridDim.x) {  // same trip count for every wave
      const int u = ub + pair;
      const bool live = u < units;
      const int j = live ? u / per_slot : 0, i0 = live ? (u - j * per_slot) * kUnitRows : 0;
      const float2 gu = unit_gate_up<2>(p.L, s_ids[j], i0, half ? gmid : 0, half ? G : gmid, xp, xs);
      if (half && (lane & 7) == 0) s_pair[pair][lane >> 3] = gu;
      __syncthreads();
      if (!half && live) {
        const float2 o = s_pair[pair][lane >> 3];
        const float g = gu.x + o.x, up = gu.y + o.y;
        publish_unit(p.act + (size_t)j * I, i0, I, silu(g) * up, epoch);
      }
      __syncthreads();
    }
  }

  // prefetch the down rows this workgroup owns in phase C (its first row block);
  // issued after phase B's loads so they do not compete with them, and hidden
  // behind the activation handoff
  const int LI = 1 << p.lsI, subI = lane & (LI - 1), rsubI = lane >> p.lsI, rpiI = kWave >> p.lsI;
  const int GI = I >> 6;
  const bool pf_ok = GI == LI && (int)blockIdx.x * rpiI < H;
  DownPrefetch pf[kPrefetchSlots];
  // an 8-bit shared expert: the down-row group of this lane for the first row block,
  // held by the wave that takes the shared slot (slot k, wave k % kWaves)
  uint4 qpf[4] = {};
  uint32_t qps = 0, qpb = 0;
  if constexpr (kQ8Shared) {
    const int n = blockIdx.x * rpiI + rsubI;
    if (pf_ok && k % kWaves == wv && n < H) {
      const uint4* cr = reinterpret_cast<const uint4*>(p.L.sh_down.codes) + (int64_t)n * (I >> 4) + 4 * subI;
#pragma unroll
      for (int q = 0; q < 4; ++q) qpf[q] = cr[q];
      qps = p.L.sh_down.scales[(int64_t)n * GI + subI];
      qpb = p.L.sh_down.biases[(int64_t)n * GI + subI];
    }
  }
  {
    const int n = blockIdx.x * rpiI + rsubI;
    const int64_t mat_codes = (int64_t)H * (I >> 3), mat_groups = (int64_t)H * GI;
#pragma unroll
    for (int s = 0; s < kPrefetchSlots; ++s) {
      const int j = wv + kWaves * s;
      if (pf_ok && j < nslot && n < H && !(kQ8Shared && s_ids[j] < 0)) {
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

  // ------------------------------------------------------------ phase C
  // routed slots and the shared slot (an 8-bit shared expert's slot also as fp32 into af)
  stage_tagged_split(p.act, nslot, I, ap, as, epoch, timeouts, kQ8Shared ? af : nullptr, k * I);
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
          if (kQ8Shared && e < 0 && first) {
            part = q8_group_term_regs(qpf, af + subI * kQ8Pad, qps, qpb);  // one group per lane (GI == LI)
          } else if (kQ8Shared && e < 0) {
            const uint4* cr = reinterpret_cast<const uint4*>(p.L.sh_down.codes) + (int64_t)n * (I >> 4);
            const uint16_t* sr = p.L.sh_down.scales + (int64_t)n * GI;
            const uint16_t* br = p.L.sh_down.biases + (int64_t)n * GI;
            for (int g = subI; g < GI; g += LI) part += q8_group_term(cr + 4 * g, af + g * kQ8Pad, sr[g], br[g]);
          } else if (first && s < kPrefetchSlots) {
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
          if (p.out_mode == kOutBf16Residual) t += bf16_bits_to_f32(p.x[nn]);
          if (p.out_mode != kOutF32)
            reinterpret_cast<uint16_t*>(p.y)[nn] = (uint16_t)f32_to_bf16_bits(t);
          else
            reinterpret_cast<float*>(p.y)[nn] = t;
        }
      }
      __syncthreads();
    }
  }
}

#define Q4MOE_DECODE_KERNEL(name, q8r, gated, q8sh) \
  __global__ __launch_bounds__(kThreads) void name(DecodeParams p) { decode_layer<q8r, gated, q8sh>(p); }
Q4MOE_DECODE_KERNEL(decode_layer_kernel, false, false, false)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_kernel, true, false, false)
Q4MOE_DECODE_KERNEL(decode_layer_gated_kernel, false, true, false)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_gated_kernel, true, true, false)
Q4MOE_DECODE_KERNEL(decode_layer_q8shared_kernel, false, false, true)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_q8shared_kernel, true, false, true)
Q4MOE_DECODE_KERNEL(decode_layer_gated_q8shared_kernel, false, true, true)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_gated_q8shared_kernel, true, true, true)
#undef Q4MOE_DECODE_KERNEL

int lanes_log2(int groups) {
  int r = 0;
  while (r < 6 && (2 << r) <= groups) ++r;
  return r;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t decode_lds(const DecodeLayer& L) {
  const int nslot = L.top_k + (L.has_shared ? 1 : 0);
  size_t b = (size_t)(L.hidden >> 5) * (chunk_stride<1>() * 4 + 4) +
             (size_t)nslot * (L.inter >> 5) * (chunk_stride<2>() * 4 + 4);
  if (L.has_shared && L.sh_q8) b += 16 + (size_t)((L.hidden >> 6) + (L.inter >> 6)) * kQ8Pad * 4;
  return b;
}

}  // namespace

size_t decode_workspace_bytes(int hidden, int inter, int n_experts, int top_k) {
  (void)hidden;
  (void)n_experts;
  return align256(sizeof(DecodeWs)) + align256((size_t)(top_k + 1) * inter * 8);
}

size_t decode_lds_bytes(const DecodeLayer& L) { return decode_lds(L); }

hipError_t run_moe_ffn_decode(const DecodeLayer& L, const uint16_t* x, void* y, int out_mode, int32_t* ids_out,
                              float* w_out, void* ws, hipStream_t stream) {
  DecodeParams p{};
  p.L = L;
  p.x = x;
  p.y = y;
  p.out_mode = out_mode;
  p.ids_out = ids_out;
  p.w_out = w_out;
  char* w = static_cast<char*>(ws);
  p.ws = reinterpret_cast<DecodeWs*>(w);
  w += align256(sizeof(DecodeWs));
  p.act = reinterpret_cast<unsigned long long*>(w);
  p.lsH = lanes_log2(L.hidden / kGroup);
  p.lsI = lanes_log2(L.inter / kGroup);
  const size_t lds = decode_lds(L);
  int blocks = device_cu_count();
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  typedef void (*Kernel)(DecodeParams);
  static const Kernel kernels[2][2][2] = {
      {{decode_layer_kernel, decode_layer_q8shared_kernel}, {decode_layer_gated_kernel, decode_layer_gated_q8shared_kernel}},
      {{decode_layer_q8router_kernel, decode_layer_q8router_q8shared_kernel},
       {decode_layer_q8router_gated_kernel, decode_layer_q8router_gated_q8shared_kernel}}};
  const int q8 = L.router_q8.codes != nullptr, gated = L.sh_gate_w != nullptr && L.has_shared,
            q8sh = L.has_shared && L.sh_q8;
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernels[q8][gated][q8sh]), dim3(blocks),
                                       dim3(kThreads), args, lds, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace q4moe
