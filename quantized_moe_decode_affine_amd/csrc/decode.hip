// Batch-1 decode step of one MoE feed-forward layer in one launch.
//
// The step is a dependent chain of weight streams (lily-qwen3.8-flash-next
// README, "How the speed was achieved": decode is bandwidth-bound and its
// kernels are tuned against the chain of reads).  One grid of one workgroup
// per CU keeps that chain as short as it can be: three weight streams and two
// handoffs between workgroups.
//   A: every workgroup reads its router row(s) (one 4 KB row for 256 experts on
//      256 CUs) and publishes the logit; meanwhile it issues the loads of the
//      shared expert's gate/up rows it owns (they depend on nothing) and
//      computes them with SwiGLU after the logit is out.
//   B: every workgroup takes the top-k itself from the published logits, then
//      issues at once every routed weight it will need in this launch: its
//      gate/up rows AND the down rows of the output rows it owns (the down
//      rows depend only on the expert ids, not on the activations), so the
//      down stream is in flight while gate/up is computed and handed over.
//   C: the SwiGLU activations of every slot are staged into LDS and the
//      already-loaded down rows are reduced; each output row is combined in a
//      fixed slot order (no atomics), y written once.
//
// No grid-wide barrier: every value handed from one workgroup to another (the
// router logits, the SwiGLU activations) is one 64-bit word {epoch, fp32 bits}
// written by one store of this launch, so a consumer's load both reads the value
// and tells whether it is there yet; only late words are polled again.  Because
// the value travels inside the flag word, no ordering between two memory
// locations is needed: the handoff relies only on the single-copy atomicity of
// an aligned 64-bit store and on device-coherent (L2-bypassing) loads.  The 8
// words of an activation line are written by one store instruction.  The epoch
// is agreed through per-group arrival counters in the workspace.  Every poll is
// bounded: a lost flag yields a wrong result and a recorded timeout, never a hang.
#include "handoff.h"
#include "kernels.h"
#include "topk.h"
#include "vecstage.h"

#include <mutex>

namespace q4moe {

namespace {

#ifndef Q4MOE_DECODE_THREADS
#define Q4MOE_DECODE_THREADS 512
#endif
constexpr int kThreads = Q4MOE_DECODE_THREADS;
constexpr int kWaves = kThreads / kWave;

constexpr int kMaxBlocks = 1024;
constexpr int kOutRows = 8;       // output rows of one down block
constexpr int kUnitRows = 8;      // gate/up row pairs of one unit: one 64-byte line of activations
constexpr int kGuSlots = 1024 / kThreads;  // routed gate/up row pairs per lane loaded at top-k time (16 pairs per CU)
constexpr int kShSlots = 512 / kThreads;   // shared gate/up row pairs per lane loaded at launch (8 pairs per CU)
constexpr int kDnSlots = 1536 / kThreads;  // down rows per lane loaded at top-k time (96 rows of 16 lanes per CU)
constexpr int kRtRows = 2;        // router rows per workgroup whose loads go out at launch
constexpr int kActBatch = 256;    // activations gathered in LDS before they are published
#ifndef Q4MOE_DOWN_LATE
#define Q4MOE_DOWN_LATE 0
#endif
constexpr bool kDownLate = Q4MOE_DOWN_LATE;  // down rows loaded after gate/up (else with it)
#ifndef Q4MOE_DOWN_AFTER_GU
#define Q4MOE_DOWN_AFTER_GU 1
#endif
// down rows issued once this wave's routed gate/up rows are in (they are needed only
// after the activation handoff; issued with the gate/up rows they share the stream)
constexpr bool kDownAfterGu = Q4MOE_DOWN_AFTER_GU;
#ifndef Q4MOE_SHARED_LATE
#define Q4MOE_SHARED_LATE 1
#endif
constexpr bool kSharedLate = Q4MOE_SHARED_LATE;  // shared gate/up rows issued after the router rows are in

#ifndef Q4MOE_HANDOFF_COPIES
#define Q4MOE_HANDOFF_COPIES 8
#endif
#ifndef Q4MOE_LOGIT_STRIDE
#define Q4MOE_LOGIT_STRIDE 1
#endif
constexpr int kLogitStride = Q4MOE_LOGIT_STRIDE;  // 64-bit words per logit slot
// Every value handed between workgroups is written to kCopies copies, and workgroup b
// reads copy b % kCopies: the copies sit on different memory channels, so the reads of
// all workgroups do not queue at the few channels that would hold a single copy.
constexpr int kCopies = Q4MOE_HANDOFF_COPIES;
constexpr int kLogitCopyWords = kMaxExperts * kLogitStride + 64;  // words between logit copies (skewed)

// Phase stamps, in a diagnostic build only (-DQ4MOE_DECODE_STAMPS: build.py --stamps
// writes it to a library file of its own): thread 0 of every workgroup records the
// 100 MHz s_memrealtime counter at the layer's phase boundaries, slot (epoch % 4) of the
// array, so the last four launches can be read back (q4moe_decode_stamps below).
// Stamps: 0 launch start, 1 router logits published, 2 top-k known, 3 gate/up computed,
// 4 activations staged, 5 end.
#ifdef Q4MOE_DECODE_STAMPS
__device__ unsigned long long g_decode_stamps[4][kMaxBlocks][8];
#define Q4MOE_STAMP(i, v)                                                                   \
  do {                                                                                     \
    if (threadIdx.x == 0) g_decode_stamps[s_epoch & 3][blockIdx.x][i] = (v);               \
  } while (0)
#else
#define Q4MOE_STAMP(i, v) \
  do {                    \
  } while (0)
#endif

struct DecodeWs {
  HandoffHead h;  // epoch counters; the timeout count at byte 2048
  // Router logit of expert e: tag_logit[e * kLogitStride] = {epoch:hi32, fp32 bits:lo32}.
  // Each logit has a 64-byte line of its own: a line written by several workgroups
  // is observed several times more slowly than one written by a single store.
  unsigned long long tag_logit[kCopies * kLogitCopyWords];
};

struct DecodeParams {
  const uint16_t* x;          // [H]
  void* y;                    // [H]
  int out_mode;               // kOutF32, kOutBf16, kOutBf16Residual
  int32_t* ids_out;           // nullable [k]
  float* w_out;               // nullable [k]
  DecodeWs* ws;
  unsigned long long* act;    // kCopies x [k+1][I] tagged SwiGLU outputs: routed slots 0..k-1, shared slot k
  int64_t act_copy_words;     // words between the copies of act
  DecodeLayer L;              // last: the per-call fields above keep fixed small offsets
};

int lanes_log2(int n) {
  int r = 0;
  while (r < 6 && (2 << r) <= n) ++r;
  return r;
}

__device__ __forceinline__ int dev_lanes_log2(int n) {
  int r = 0;
  while (r < 6 && (2 << r) <= n) ++r;
  return r;
}

// Stage a bf16 vector of n values (n % 32 == 0) into LDS as permuted pairs with
// chunk sums: each thread takes one 8-value block per pass, chunk sums by a quad
// reduction (the 4 blocks of a chunk sit in one lane quad).
__device__ __forceinline__ void stage_bf16_parallel(const uint16_t* __restrict__ x, int n, uint32_t* vp, float* vs) {
  constexpr int ST = chunk_stride<1>();
  const int t = threadIdx.x;
  const int nblk = n >> 3;
  for (int base = 0; base < nblk; base += kThreads) {
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

// Stage block b (8 values held in v) of a bf16 vector of nblk blocks into LDS: every
// thread of the workgroup calls this with its own block (b >= nblk: nothing stored);
// chunk sums by a quad reduction (the 4 blocks of a chunk sit in one lane quad).
__device__ __forceinline__ void stage_bf16_block(uint4 v, int b, int nblk, uint32_t* vp, float* vs) {
  constexpr int ST = chunk_stride<1>();
  float sum = (bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16)) +
              (bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16)) +
              (bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16)) +
              (bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16));
  if (b < nblk) *reinterpret_cast<uint4*>(vp + (b >> 2) * ST + (b & 3) * 4) = permute_block(v);
  sum = group_sum_rt(sum, 2);
  if (b < nblk && (b & 3) == 0) vs[b >> 2] = sum;
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
constexpr int kTagRounds = (4608 + 2 * kThreads - 1) / (2 * kThreads);  // 16-byte loads per thread: 9 slots x 512 words in one pass

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
    // every pair still incomplete is fetched again, all of them in flight together, so a
    // poll costs one round trip however many words are late
    for (unsigned spins = 0;; ++spins) {
      bool done = true;
#pragma unroll
      for (int r = 0; r < kTagRounds; ++r) done &= base + r * nthr + t >= npairs || complete(r);
      if (__all(done)) break;
      if (spins == kPollLimit) {
        if (lane_id() == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int r = 0; r < kTagRounds; ++r)
        if (!(base + r * nthr + t >= npairs || complete(r))) fetch(r);
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

// ------------------------------------------------------------ row tasks
//
// A row of C chunks (32 codes, one 16-byte word each) is taken by LR = 2^lr
// consecutive lanes (lr = lanes_log2(C), at most 64): lane `sub` of the group
// takes chunks sub, sub + LR, ...  A wave covers RPW = 64 / LR rows per pass and
// the workgroup kWaves * RPW rows.  When C is a power of two no larger than 64 a
// lane holds exactly one chunk of every row it takes (the form whose loads can be
// issued ahead into registers).
struct RowGeom {
  int lr, LR, RPW, sub, lg, C;
  bool one;  // one chunk per lane per row
};

__device__ __forceinline__ RowGeom row_geom(int C) {
  RowGeom g;
  g.C = C;
  g.lr = dev_lanes_log2(C);
  g.LR = 1 << g.lr;
  g.RPW = kWave >> g.lr;
  const int lane = lane_id();
  g.sub = lane & (g.LR - 1);
  g.lg = lane >> g.lr;
  g.one = g.LR == C;
  return g;
}

// One gate/up row pair (intermediate row i) of routed expert e, or of the shared expert.
struct PairRef {
  const uint4* gc;
  const uint4* uc;
  const uint16_t *gs, *gb, *us, *ub;
};

__device__ __forceinline__ PairRef make_pair_ref(const uint32_t* gcodes, const uint16_t* gscales,
                                                 const uint16_t* gbiases, const uint32_t* ucodes,
                                                 const uint16_t* uscales, const uint16_t* ubiases, int64_t row,
                                                 int H) {
  const int C = H >> 5, G = H >> 6;
  PairRef r;
  r.gc = reinterpret_cast<const uint4*>(gcodes) + row * C;
  r.uc = reinterpret_cast<const uint4*>(ucodes) + row * C;
  r.gs = gscales + row * G;
  r.gb = gbiases + row * G;
  r.us = uscales + row * G;
  r.ub = ubiases + row * G;
  return r;
}

__device__ __forceinline__ PairRef routed_pair_ref(const DecodeLayer& L, int e, int i) {
  return make_pair_ref(L.gate.codes, L.gate.scales, L.gate.biases, L.up.codes, L.up.scales, L.up.biases,
                       (int64_t)e * L.inter + i, L.hidden);
}

__device__ __forceinline__ PairRef shared_pair_ref(const DecodeLayer& L, int i) {
  return make_pair_ref(L.sh_gate.codes, L.sh_gate.scales, L.sh_gate.biases, L.sh_up.codes, L.sh_up.scales,
                       L.sh_up.biases, i, L.hidden);
}

// The codes, scales and biases of one chunk of a gate/up row pair, loaded ahead.
struct PairRegs {
  uint4 g, u;
  uint32_t gs, gb, us, ub;
};

__device__ __forceinline__ void load_pair(const PairRef& r, int c, PairRegs& d) {
  d.g = r.gc[c];
  d.u = r.uc[c];
  d.gs = r.gs[c >> 1];
  d.gb = r.gb[c >> 1];
  d.us = r.us[c >> 1];
  d.ub = r.ub[c >> 1];
}

// One chunk (32 codes, 32 bytes per matrix) of a gate/up row pair of an 8-bit shared
// expert ([I][H/4] words), loaded ahead.
struct PairRegs8 {
  uint4 g0, g1, u0, u1;
  uint32_t gs, gb, us, ub;
};

__device__ __forceinline__ void load_pair8(const DecodeLayer& L, int64_t row, int c, PairRegs8& d) {
  const int H = L.hidden, G = H >> 6;
  const uint4* gc = reinterpret_cast<const uint4*>(L.sh_gate.codes) + row * (H >> 4) + 2 * c;
  const uint4* uc = reinterpret_cast<const uint4*>(L.sh_up.codes) + row * (H >> 4) + 2 * c;
  d.g0 = gc[0];
  d.g1 = gc[1];
  d.u0 = uc[0];
  d.u1 = uc[1];
  d.gs = L.sh_gate.scales[row * G + (c >> 1)];
  d.gb = L.sh_gate.biases[row * G + (c >> 1)];
  d.us = L.sh_up.scales[row * G + (c >> 1)];
  d.ub = L.sh_up.biases[row * G + (c >> 1)];
}

// The 16 pair words of a staged bf16 chunk, read once from LDS.
struct XChunk {
  uint32_t v[16];
  float sum;
};

__device__ __forceinline__ void read_xchunk(const uint32_t* xp, const float* xs, int c, XChunk& x) {
  const uint32_t* src = xp + c * chunk_stride<1>();
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint4 t = *reinterpret_cast<const uint4*>(src + 4 * b);
    x.v[4 * b] = t.x;
    x.v[4 * b + 1] = t.y;
    x.v[4 * b + 2] = t.z;
    x.v[4 * b + 3] = t.w;
  }
  x.sum = xs[c];
}

__device__ __forceinline__ float chunk_pdot_regs(uint4 codes, const uint32_t (&v)[16]) {
  float p0 = word_dot(codes.x, v + 0, 0.f);
  float p1 = word_dot(codes.y, v + 4, 0.f);
  p0 = word_dot(codes.z, v + 8, p0);
  p1 = word_dot(codes.w, v + 12, p1);
  return p0 + p1;
}

// (gate, up) partial of one chunk.
__device__ __forceinline__ float2 pair_terms(const PairRegs& d, const XChunk& x) {
  return make_float2(affine_term(chunk_pdot_regs(d.g, x.v), x.sum, d.gs, d.gb),
                     affine_term(chunk_pdot_regs(d.u, x.v), x.sum, d.us, d.ub));
}

// (gate, up) partial of one chunk of an 8-bit pair: 8-bit codes are exact bf16 values,
// so a group contributes scale * sum(q x) + bias * sum(x).
__device__ __forceinline__ float2 pair_terms8(const PairRegs8& d, const XChunk& x) {
  return make_float2(fmaf(bf16_bits_to_f32(d.gs), q8_chunk_pdot_regs(d.g0, d.g1, x.v), bf16_bits_to_f32(d.gb) * x.sum),
                     fmaf(bf16_bits_to_f32(d.us), q8_chunk_pdot_regs(d.u0, d.u1, x.v), bf16_bits_to_f32(d.ub) * x.sum));
}

// Full (gate, up) dots of a row pair by the lane group, loads issued on the spot
// (chunks sub, sub + LR, ...); every lane of the group returns the totals.
__device__ __forceinline__ float2 pair_dot_now(const PairRef& r, const RowGeom& g, const uint32_t* xp,
                                               const float* xs, bool live) {
  float ag = 0.f, au = 0.f;
  for (int c = g.sub; c < g.C; c += g.LR) {  // lanes past C idle
    if (live) {
      PairRegs d;
      load_pair(r, c, d);
      XChunk x;
      read_xchunk(xp, xs, c, x);
      const float2 t = pair_terms(d, x);
      ag += t.x;
      au += t.y;
    }
  }
  return make_float2(group_sum_rt(ag, g.lr), group_sum_rt(au, g.lr));
}

// ------------------------------------------------------------ 8-bit shared expert
// An 8-bit shared expert (affine Q8, code j of a row in byte j % 4 of word j / 4)
// is read against fp32 copies of its input in LDS, one 64-column group per row of
// kQ8Pad floats: the 64 values, then (for x) their sum.  Its gate/up units are 8 rows
// of 8 lanes (one group per lane at a time).
constexpr int kQ8LaneLog = 3;

template <class Get>
__device__ __forceinline__ void stage_q8_groups(float* dst, int n, Get get) {
  const int lane = lane_id();
  for (int g = threadIdx.x / kWave; g < (n >> 6); g += kWaves) {
    const float v = get(g * 64 + lane);
    dst[g * kQ8Pad + lane] = v;
    const float t = group_sum_rt(v, 6);
    if (lane == 0) dst[g * kQ8Pad + 64] = t;
  }
}

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

// scale * sum(q v) + bias * sum(v) over one 64-column group of an 8-bit row read from memory.
__device__ __forceinline__ float q8_group_term(const uint4* c, const float* v, uint32_t s, uint32_t b) {
  uint4 w4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) w4[q] = c[q];
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

// Gate/up of rows i0..i0+7 of an 8-bit shared expert over all groups: lane l takes
// row i0 + l/8 and groups l%8, l%8 + 8, ...; every lane of a row's 8-lane group
// returns that row's (g, u).  xf is the input in padded groups.
__device__ __forceinline__ float2 unit_gate_up_q8(const DecodeLayer& L, int i0, const float* xf) {
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
  for (int base = 0; base < G; base += 2 * LPR) {  // wave-uniform trip count
    const bool ok0 = base + gl < G, ok1 = base + gl + LPR < G;
    const int g0 = min(base + gl, G - 1), g1 = min(base + gl + LPR, G - 1);
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

// Down row n of an 8-bit shared expert against its fp32 activations af (padded groups):
// lanes sub, sub + LR, ... of the row's group take groups; returns the row total.
__device__ __forceinline__ float q8_down_row(const DecodeLayer& L, int n, const float* af, int sub, int LR, int lr,
                                             bool live) {
  const int I = L.inter, GI = I >> 6;
  float part = 0.f;
  if (live) {
    const uint4* cr = reinterpret_cast<const uint4*>(L.sh_down.codes) + (int64_t)n * (I >> 4);
    const uint16_t* sr = L.sh_down.scales + (int64_t)n * GI;
    const uint16_t* br = L.sh_down.biases + (int64_t)n * GI;
    for (int g = sub; g < GI; g += LR) part += q8_group_term(cr + 4 * g, af + g * kQ8Pad, sr[g], br[g]);
  }
  return group_sum_rt(part, lr);
}

// ------------------------------------------------------------ handoffs

// Publish the activations gathered in LDS (s_act[m * 8 + r] = row r of unit m) as
// tagged words, one 64-byte line per unit written by 8 lanes of one wave (the
// waves take units in turn).  unit_slot(m) returns {slot, first row} of unit m.
template <class UnitOf>
__device__ __forceinline__ void publish_units(unsigned long long* act, int64_t copy_words, int I, const float* s_act,
                                              int nunits, uint32_t epoch, UnitOf unit_of) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  for (int m = wv * 8 + (lane >> 3); m < nunits; m += kWaves * 8) {  // 8 units per wave instruction
    const int2 su = unit_of(m);
    const unsigned long long w = tag_word(epoch, s_act[m * 8 + (lane & 7)]);
    unsigned long long* dst = act + (size_t)su.x * I + su.y + (lane & 7);
#pragma unroll
    for (int c = 0; c < kCopies; ++c)
      __hip_atomic_store(dst + c * copy_words, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The layer's body, specialised on the router's format (bf16, or 8-bit affine codes), on
// a shared-expert gate (the shared expert weighted by sigmoid(sh_gate_w . x)), on the
// shared expert's code width (4 or 8 bits) and on kFast: hidden 2048 and intermediate
// 512 (the 35B-A3B layer's shape), compiled as constants, with every weight load issued
// ahead into registers (unconditionally, dead tasks reading a clamped valid address, so
// no load sits behind a branch and nothing waits for a load before its use).  Other
// shapes load each weight where it is used.
constexpr int kFastHidden = 2048, kFastInter = 512;
template <bool kQ8Router, bool kShGate, bool kQ8Shared, bool kFast>
__device__ __forceinline__ void decode_layer(const DecodeParams& p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ int32_t s_ids[kMaxTopK + 1];
  __shared__ float s_w[kMaxTopK + 1];
  __shared__ float s_rpart[kRtRows][kWaves];
  __shared__ float s_act[kActBatch];
  __shared__ float s_sh[kActBatch];
  __shared__ float s_red[(kMaxTopK + 1) * kOutRows];
  __shared__ uint32_t s_epoch;

  const DecodeLayer& L = p.L;
  // the fast form is compiled for one shape, so every row geometry below is a constant
  const int H = kFast ? kFastHidden : L.hidden, I = kFast ? kFastInter : L.inter;
  const int E = L.n_experts, k = L.top_k;
  const int CH = H >> 5, CI = I >> 5;
  const bool has_shared = L.has_shared != 0;
  const int nslot = k + (has_shared ? 1 : 0);
  const int NB = gridDim.x, b = blockIdx.x;
  uint32_t* xp = smem;                                                                // [CH][ST1]
  float* xs = reinterpret_cast<float*>(xp + CH * chunk_stride<1>());                   // [CH]
  uint32_t* ap = reinterpret_cast<uint32_t*>(xs + CH);                                // [nslot][CI][ST2]
  float* as = reinterpret_cast<float*>(ap + (size_t)nslot * CI * chunk_stride<2>());  // [nslot][CI]
  const size_t xf_off = (reinterpret_cast<const uint32_t*>(as + (size_t)nslot * CI) - smem + 3) & ~size_t(3);
  float* xf = reinterpret_cast<float*>(smem + xf_off);  // 8-bit shared expert: x as fp32 [H/64][kQ8Pad]
  float* af = xf + (size_t)(H >> 6) * kQ8Pad;           // 8-bit shared expert: its activations [I/64][kQ8Pad]
  unsigned* timeouts = &p.ws->h.timeouts;

  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int t = threadIdx.x;
#ifdef Q4MOE_DECODE_STAMPS
  const unsigned long long stamp0 = __builtin_amdgcn_s_memrealtime();
#endif

  // ---- epoch of this launch: the arrivals of one group agree on its counter's epoch
  // field.  Thread 0's arrival goes out right after the router loads; its result is
  // used after the dots.
  auto finish_epoch = [&](unsigned long long old) { s_epoch = epoch_finish(&p.ws->h, b, NB, old); };

  const RowGeom gh = row_geom(CH);
  const RowGeom gd = row_geom(CI);
  const int PS = kWaves * gh.RPW;  // gate/up row pairs per pass
  const int nbatch_units = kActBatch / kUnitRows;
  const int upe = I / kUnitRows;   // gate/up units per expert

  // ================================================================ phase A
  // Router rows e = b, b + NB, ... (one 16-byte word of a row per thread when fast).
  const int nrows_rt = b < E ? (E - 1 - b) / NB + 1 : 0;
  // Fast form: the first kRtRows rows go out now into registers (8-bit router: one
  // 16-code word of a row, with its group's scale and bias and the matching 16 values
  // of x, per thread of the first H / 16).
  constexpr bool rt_pf = kFast && !kQ8Router, rt_pf8 = kFast && kQ8Router;
  uint4 rreg[kRtRows], xreg, xq0, xq1;
  uint16_t rsc[kRtRows], rbi[kRtRows];
  if constexpr (rt_pf || rt_pf8) xreg = reinterpret_cast<const uint4*>(p.x)[min(t, (H >> 3) - 1)];
  if constexpr (rt_pf) {
    const int c = min(t, (H >> 3) - 1);
#pragma unroll
    for (int m = 0; m < kRtRows; ++m)
      rreg[m] = reinterpret_cast<const uint4*>(L.router + (size_t)min(b + m * NB, E - 1) * H)[c];
  }
  if constexpr (rt_pf8) {
    const int c = min(t, (H >> 4) - 1), G = H >> 6;
    xq0 = reinterpret_cast<const uint4*>(p.x)[2 * c];
    xq1 = reinterpret_cast<const uint4*>(p.x)[2 * c + 1];
#pragma unroll
    for (int m = 0; m < kRtRows; ++m) {
      const size_t e = (size_t)min(b + m * NB, E - 1);
      rreg[m] = reinterpret_cast<const uint4*>(L.router_q8.codes)[e * (H >> 4) + c];
      rsc[m] = L.router_q8.scales[e * G + (c >> 2)];
      rbi[m] = L.router_q8.biases[e * G + (c >> 2)];
    }
  }
  unsigned long long arrival;
  if (t == 0) arrival = epoch_arrive(&p.ws->h, b);

  // Shared gate/up units su = b, b + NB, ... (8 row pairs each): in the fast form the
  // loads of the first kShSlots passes go out into registers once the router rows are
  // in (they depend on nothing, and issued with the router rows they would only slow
  // the logits that every workgroup waits for).
  const int sh_units = has_shared && b < upe ? (upe - 1 - b) / NB + 1 : 0;
  const int sh_pairs = min(sh_units, nbatch_units) * kUnitRows;  // the first batch
  const int sh_passes = (sh_pairs + PS - 1) / PS;
  auto sh_row = [&](int P) { return (b + (P / kUnitRows) * NB) * kUnitRows + (P % kUnitRows); };
  constexpr bool sh_pf = kFast && !kQ8Shared;
  constexpr bool sh_pf8 = kFast && kQ8Shared;  // the fast form's 8-bit shared expert: same tasks, byte codes
  const int sh_pfp = sh_pf || sh_pf8 ? min(sh_passes, kShSlots) : 0;
  PairRegs shr[kShSlots];
  PairRegs8 shr8[kShSlots];
  auto issue_shared = [&]() {
  if constexpr (sh_pf8) {
    const int lastP = sh_pairs > 0 ? sh_pairs - 1 : 0;
    const int bsh = sh_pairs > 0 ? b : upe - 1;
#pragma unroll
    for (int q = 0; q < kShSlots; ++q) {
      const int P = min(q * PS + wv * gh.RPW + gh.lg, lastP);
      load_pair8(L, (int64_t)(bsh + (P / kUnitRows) * NB) * kUnitRows + (P % kUnitRows), gh.sub, shr8[q]);
    }
  }
  if constexpr (sh_pf) {
    // clamped: a workgroup without shared work reads the last unit's rows (never used)
    const int lastP = sh_pairs > 0 ? sh_pairs - 1 : 0;
    const int bsh = sh_pairs > 0 ? b : upe - 1;
#pragma unroll
    for (int q = 0; q < kShSlots; ++q) {
      const int P = min(q * PS + wv * gh.RPW + gh.lg, lastP);
      const int i = has_shared ? (bsh + (P / kUnitRows) * NB) * kUnitRows + (P % kUnitRows) : 0;
      load_pair(has_shared ? shared_pair_ref(L, i) : routed_pair_ref(L, 0, 0), gh.sub, shr[q]);
    }
  }
  };
  // (8-bit shared rows, four times the bytes of 4-bit ones on a quarter of the workgroups,
  // go out at once: issued late they would hold up phase B)
  constexpr bool sh_late = kSharedLate && !kQ8Shared;
  if (!sh_late) issue_shared();

  // Router dots, one partial per thread, then a fixed-order sum over the waves.
  for (int m0 = 0; m0 < nrows_rt; m0 += kRtRows) {
#pragma unroll
    for (int mm = 0; mm < kRtRows; ++mm) {
      const int m = m0 + mm;
      if (m >= nrows_rt) break;
      const int e = b + m * NB;
      float part = 0.f;
      if (rt_pf8 && m < kRtRows) {
        const uint32_t xw[8] = {xq0.x, xq0.y, xq0.z, xq0.w, xq1.x, xq1.y, xq1.z, xq1.w};
        const uint32_t cw[4] = {rreg[mm].x, rreg[mm].y, rreg[mm].z, rreg[mm].w};
        float pq = 0.f, xsum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float xi = bf16_bits_to_f32((xw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
          xsum += xi;
          pq = fmaf(xi, (float)((cw[i >> 2] >> (8 * (i & 3))) & 0xFFu), pq);
        }
        part = t < (H >> 4) ? fmaf(bf16_bits_to_f32(rsc[mm]), pq, bf16_bits_to_f32(rbi[mm]) * xsum) : 0.f;
      } else if constexpr (kQ8Router) {
        // 8-bit router (count 1, [E][H/4] words): 16-code chunks per thread (inside one group)
        const int G = H >> 6;
        const uint4* qr = reinterpret_cast<const uint4*>(L.router_q8.codes) + (size_t)e * (H >> 4);
        const uint4* xv = reinterpret_cast<const uint4*>(p.x);
        for (int c = t; c < (H >> 4); c += kThreads) {
          const uint4 w = qr[c], xa = xv[2 * c], xb = xv[2 * c + 1];
          const float sc = bf16_bits_to_f32(L.router_q8.scales[(size_t)e * G + (c >> 2)]);
          const float o = bf16_bits_to_f32(L.router_q8.biases[(size_t)e * G + (c >> 2)]);
          const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
          const uint32_t cw[4] = {w.x, w.y, w.z, w.w};
          float pq = 0.f, xsum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float xi = bf16_bits_to_f32((xw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
            xsum += xi;
            pq = fmaf(xi, (float)((cw[i >> 2] >> (8 * (i & 3))) & 0xFFu), pq);
          }
          part += fmaf(sc, pq, o * xsum);
        }
      } else if (rt_pf && m < kRtRows) {
        const uint4 w = rreg[mm];
        float a0 = dot2_bf16(w.x, xreg.x, 0.f), a1 = dot2_bf16(w.y, xreg.y, 0.f);
        a0 = dot2_bf16(w.z, xreg.z, a0);
        a1 = dot2_bf16(w.w, xreg.w, a1);
        part = t < (H >> 3) ? a0 + a1 : 0.f;
      } else {
        const uint4* rr = reinterpret_cast<const uint4*>(L.router + (size_t)e * H);
        const uint4* xv = reinterpret_cast<const uint4*>(p.x);
        float a0 = 0.f, a1 = 0.f;
        for (int c = t; c < (H >> 3); c += kThreads) {
          const uint4 w = rr[c], v = xv[c];
          a0 = dot2_bf16(w.x, v.x, a0);
          a1 = dot2_bf16(w.y, v.y, a1);
          a0 = dot2_bf16(w.z, v.z, a0);
          a1 = dot2_bf16(w.w, v.w, a1);
        }
        part = a0 + a1;
      }
      part = group_sum_rt(part, 6);
      if (lane == 0) s_rpart[mm][wv] = part;
    }
    if constexpr (rt_pf || rt_pf8) {
      if (m0 == 0) stage_bf16_block(xreg, t, H >> 3, xp, xs);  // x from the router pass's registers
    }
    if (t == 0 && m0 == 0) finish_epoch(arrival);
    lds_sync();  // partials (and, on the first pass, the epoch) visible
#ifdef Q4MOE_DECODE_STAMPS
    if (m0 == 0) {
      Q4MOE_STAMP(0, stamp0);
      Q4MOE_STAMP(1, __builtin_amdgcn_s_memrealtime());
    }
#endif
    if (t < kRtRows * kCopies && m0 + t / kCopies < nrows_rt) {  // one thread per (row, copy)
      const int mm = t / kCopies, c = t % kCopies;
      float v = s_rpart[mm][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += s_rpart[mm][w];
      __hip_atomic_store(&p.ws->tag_logit[(size_t)c * kLogitCopyWords + (size_t)(b + (m0 + mm) * NB) * kLogitStride],
                         tag_word(s_epoch, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lds_sync();  // s_rpart is reused
  }
  if (t == 0 && nrows_rt == 0) finish_epoch(arrival);
  if (!(rt_pf || rt_pf8) || nrows_rt == 0) {
    stage_bf16_parallel(p.x, H, xp, xs);
    lds_sync();  // x staged; the epoch is visible
  }
  if constexpr (kQ8Shared && !kFast) {
    stage_q8_groups(xf, H, [&](int i) { return bf16_bits_to_f32(p.x[i]); });
    lds_sync();
  }
  if (sh_late) issue_shared();
  const uint32_t epoch = s_epoch;

  // Shared expert gate/up with SwiGLU (off the critical path: needed only in phase C),
  // into s_sh.  Waves 1.. take their share while wave 0 takes the top-k; wave 0 takes
  // its share once the routed loads are out.
  auto shared_compute = [&]() {
    if (!has_shared) return;
    if constexpr (sh_pf8) {
      XChunk x1;
      read_xchunk(xp, xs, gh.sub, x1);
#pragma unroll
      for (int q = 0; q < kShSlots; ++q) {
        if (q < sh_pfp) {
          const int P = q * PS + wv * gh.RPW + gh.lg;
          const float2 tt = pair_terms8(shr8[q], x1);
          const float g = group_sum_rt(tt.x, gh.lr), u = group_sum_rt(tt.y, gh.lr);
          if (gh.sub == 0 && P < sh_pairs) s_sh[P] = silu(g) * u;
        }
      }
      for (int q = sh_pfp; q < sh_passes; ++q) {  // (more passes than prefetched: loaded now)
        const int P = q * PS + wv * gh.RPW + gh.lg;
        PairRegs8 d;
        load_pair8(L, sh_row(min(P, sh_pairs - 1)), gh.sub, d);
        const float2 tt = pair_terms8(d, x1);
        const float g = group_sum_rt(tt.x, gh.lr), u = group_sum_rt(tt.y, gh.lr);
        if (gh.sub == 0 && P < sh_pairs) s_sh[P] = silu(g) * u;
      }
    } else if constexpr (kQ8Shared) {
      // 8-row units, one per wave at a time, on waves 1..
      for (int m = wv - 1; m >= 0 && m < min(sh_units, nbatch_units); m += kWaves - 1) {
        const float2 gu = unit_gate_up_q8(L, (b + m * NB) * kUnitRows, xf);
        if ((lane & 7) == 0) s_sh[m * kUnitRows + (lane >> 3)] = silu(gu.x) * gu.y;
      }
    } else {
      if constexpr (sh_pf) {
        XChunk x1;
        read_xchunk(xp, xs, gh.sub, x1);
#pragma unroll
        for (int q = 0; q < kShSlots; ++q) {
          if (q < sh_pfp) {
            const int P = q * PS + wv * gh.RPW + gh.lg;
            const float2 tt = pair_terms(shr[q], x1);
            const float g = group_sum_rt(tt.x, gh.lr), u = group_sum_rt(tt.y, gh.lr);
            if (gh.sub == 0 && P < sh_pairs) s_sh[P] = silu(g) * u;
          }
        }
      }
      for (int q = sh_pfp; q < sh_passes; ++q) {
        const int P = q * PS + wv * gh.RPW + gh.lg;
        const bool live = P < sh_pairs;
        const float2 gu = pair_dot_now(shared_pair_ref(L, live ? sh_row(P) : 0), gh, xp, xs, live);
        if (gh.sub == 0 && live) s_sh[P] = silu(gu.x) * gu.y;
      }
    }
  };
  if (wv != 0) shared_compute();

  if (wv == 0) {
    // The shared expert's gate, sigmoid(sh_gate_w . x), taken while the router logits of the
    // other workgroups are still arriving (the top-k below waits for them).
    float sh_weight = 1.0f;
    if constexpr (kShGate) {
      const uint4* gw = reinterpret_cast<const uint4*>(L.sh_gate_w);
      const uint4* gx = reinterpret_cast<const uint4*>(p.x);
      float d0 = 0.f, d1 = 0.f;
      for (int c = lane; c < (H >> 3); c += kWave) {
        const uint4 a = gw[c], bb = gx[c];
        d0 = dot2_bf16(a.x, bb.x, d0);
        d1 = dot2_bf16(a.y, bb.y, d1);
        d0 = dot2_bf16(a.z, bb.z, d0);
        d1 = dot2_bf16(a.w, bb.w, d1);
      }
      const float d = group_sum_rt(d0 + d1, 6);
      sh_weight = 1.0f / (1.0f + __expf(-d));
    }
    // B: top-k from the tagged logits (every workgroup, redundantly)
    if (E <= 4 * kWave)
      wave_topk_tagged<4, kLogitStride>(p.ws->tag_logit + (size_t)(b % kCopies) * kLogitCopyWords, E, k, epoch, timeouts, s_ids, s_w, b == 0 ? p.ids_out : nullptr,
                          b == 0 ? p.w_out : nullptr);
    else
      wave_topk_tagged<kMaxExperts / kWave, kLogitStride>(p.ws->tag_logit + (size_t)(b % kCopies) * kLogitCopyWords, E, k, epoch, timeouts, s_ids, s_w,
                                            b == 0 ? p.ids_out : nullptr, b == 0 ? p.w_out : nullptr);
    if (lane == 0 && has_shared) {
      s_ids[k] = -1;
      s_w[k] = sh_weight;
    }
  }
  lds_sync();  // ids known; shared activations gathered
  Q4MOE_STAMP(2, __builtin_amdgcn_s_memrealtime());

  // ================================================================ phase B
  // Routed gate/up units u = b, b + NB, ... of the k * I / 8 units (slot u / upe, rows
  // (u % upe) * 8 ..) and this workgroup's 8-row output blocks of the down
  // projection, for every slot.  Fast form: the loads of the first kGuSlots gate/up
  // passes and kDnSlots down passes go out now, all at once.
  const int U = k * upe;
  const int my_units = b < U ? (U - 1 - b) / NB + 1 : 0;
  auto unit_of = [&](int m) -> int2 {
    const int u = min(b + m * NB, U - 1);
    return make_int2(u / upe, (u % upe) * kUnitRows);
  };
  const int pairs0 = min(my_units, nbatch_units) * kUnitRows;
  const int passes0 = (pairs0 + PS - 1) / PS;
  const int gu_pfp = kFast ? min(passes0, kGuSlots) : 0;
  const int GI = I >> 6;
  const int PSd = kWaves * gd.RPW;
  const int dtasks = nslot * kOutRows;
  const int dpasses = (dtasks + PSd - 1) / PSd;
  const int nblocks = H / kOutRows;
  // Fast form: the k routed slots' rows of the output block are k * 8 tasks of one
  // 16-lane row chunk each, PSd a pass, the first kDnSlots passes prefetched; the shared
  // expert's 8 rows take one pass more, row r on wave r over its 64 lanes (8 columns a
  // lane), so no pass has dead tasks for k = 8 and no wave branches between row kinds.
  const int dtasks_r = k * kOutRows;
  const int dpasses_r = (dtasks_r + PSd - 1) / PSd;
  const int dn_pfp = kFast && b < nblocks ? min(dpasses_r, kDnSlots) : 0;
  const int64_t dmat_rows = (int64_t)H;
  // Down task -> {slot, row}.  With a shared expert its 8 rows sit every shs tasks from
  // task 0 (for hidden 2048 / inter 512: the first task of every wave in the first pass,
  // row r on wave r, so its heavier 8-bit rows do not pile onto two waves); the routed
  // (slot, row) pairs fill the other tasks in order.
  static_assert(kOutRows == kWaves, "one shared down row per wave");
  const int shs = max(1, min(gd.RPW, dtasks / kOutRows));  // shared rows every shs tasks (all live)
  auto task_jr = [&](int task) -> int2 {
    if (!has_shared) return make_int2(task / kOutRows, task % kOutRows);
    if (task < kOutRows * shs && task % shs == 0) return make_int2(k, task / shs);
    const int i = task - min(kOutRows, (task + shs - 1) / shs);
    return make_int2(i / kOutRows, i % kOutRows);
  };
  // down row n of slot j: its code row, scales and biases (routed expert s_ids[j], or shared)
  // The shared expert's down rows are addressed from the routed stack's base by their
  // element distance, so a row pointer is one base plus a selected offset (a select
  // between two pointers would become a per-lane load of the selected argument field).
  const int64_t sh_dc = has_shared ? (int64_t)((uintptr_t)L.sh_down.codes - (uintptr_t)L.down.codes) / 4 : 0;
  const int64_t sh_ds = has_shared ? (int64_t)((uintptr_t)L.sh_down.scales - (uintptr_t)L.down.scales) / 2 : 0;
  const int64_t sh_db = has_shared ? (int64_t)((uintptr_t)L.sh_down.biases - (uintptr_t)L.down.biases) / 2 : 0;
  auto down_row = [&](int j, int n, const uint4*& cr, const uint16_t*& sr, const uint16_t*& br) {
    const int e = s_ids[j];
    const bool routed = e >= 0;
    const int64_t row = routed ? (int64_t)e * dmat_rows + n : (int64_t)n;
    cr = reinterpret_cast<const uint4*>(L.down.codes + (routed ? 0 : sh_dc) + row * (I >> 3));
    sr = L.down.scales + (routed ? 0 : sh_ds) + row * GI;
    br = L.down.biases + (routed ? 0 : sh_db) + row * GI;
  };
  PairRegs gur[kGuSlots];
  if constexpr (kFast) {
    const int lastP = pairs0 > 0 ? pairs0 - 1 : 0;
#pragma unroll
    for (int q = 0; q < kGuSlots; ++q) {
      const int P = min(q * PS + wv * gh.RPW + gh.lg, lastP);
      const int2 su = unit_of(P / kUnitRows);
      load_pair(routed_pair_ref(L, s_ids[su.x], su.y + P % kUnitRows), gh.sub, gur[q]);
    }
  }
  struct DnRegs {  // one routed row chunk: 32 codes, its group's scale and bias
    uint4 c;
    uint32_t s, bb;
  };
  struct ShDnRegs {  // 8 columns of a shared row: 8 codes (4- or 8-bit), scale, bias
    uint2 c;
    uint32_t s, bb;
  };
  auto load_dn = [&](int q, int rb, DnRegs& d) {  // routed task of pass q (dead tasks read a valid row)
    const int task = min(q * PSd + wv * gd.RPW + gd.lg, dtasks_r - 1);
    const int64_t row = (int64_t)s_ids[task / kOutRows] * dmat_rows + rb * kOutRows + task % kOutRows;
    d.c = reinterpret_cast<const uint4*>(L.down.codes + row * (I >> 3))[gd.sub];
    d.s = L.down.scales[row * GI + (gd.sub >> 1)];
    d.bb = L.down.biases[row * GI + (gd.sub >> 1)];
  };
  auto load_shdn = [&](int rb, ShDnRegs& d) {  // shared row rb * 8 + wv, lane's 8 columns
    const int64_t n = (int64_t)rb * kOutRows + wv;
    if constexpr (kQ8Shared)
      d.c = reinterpret_cast<const uint2*>(L.sh_down.codes + n * (I >> 2))[lane];
    else
      d.c = make_uint2(L.sh_down.codes[n * (I >> 3) + lane], 0u);
    d.s = L.sh_down.scales[n * GI + (lane >> 3)];
    d.bb = L.sh_down.biases[n * GI + (lane >> 3)];
  };
  DnRegs dnr[kDnSlots];
  ShDnRegs shdn;
  auto issue_down = [&]() {
    if constexpr (!kFast) return;
    const int rb0 = min(b, nblocks - 1);
#pragma unroll
    for (int q = 0; q < kDnSlots; ++q) load_dn(q, rb0, dnr[q]);
    if (has_shared) load_shdn(rb0, shdn);
  };
  if (!kDownLate && !kDownAfterGu) issue_down();

  // gate/up with SwiGLU, gathered per batch of units in LDS, then published; the
  // shared units of phase A go out with the first batch
  for (int m0 = 0; m0 < max(my_units, 1); m0 += nbatch_units) {
    const int nm = min(nbatch_units, my_units - m0);
    const int np = max(nm, 0) * kUnitRows;
    const int npass = (np + PS - 1) / PS;
    if (m0 == 0 && wv == 0) shared_compute();  // wave 0's share of the shared expert, loads already out
    int q0 = 0;
    if constexpr (kFast) {
      if (m0 == 0) {
        if constexpr (kDownAfterGu && !kDownLate) {
          wait_vmem();  // this wave's gate/up rows (and everything before them) are in
          issue_down();
        }
        XChunk x1;
        read_xchunk(xp, xs, gh.sub, x1);
#pragma unroll
        for (int q = 0; q < kGuSlots; ++q) {
          if (q < gu_pfp) {
            const int P = q * PS + wv * gh.RPW + gh.lg;
            const float2 tt = pair_terms(gur[q], x1);
            const float g = group_sum_rt(tt.x, gh.lr), u = group_sum_rt(tt.y, gh.lr);
            if (gh.sub == 0 && P < np) s_act[P] = silu(g) * u;
          }
        }
        q0 = gu_pfp;
      }
    }
    for (int q = q0; q < npass; ++q) {
      const int P = q * PS + wv * gh.RPW + gh.lg;
      const bool live = P < np;
      const int2 su = unit_of(m0 + (live ? P / kUnitRows : 0));
      const float2 gu =
          pair_dot_now(routed_pair_ref(L, s_ids[su.x], su.y + (live ? P % kUnitRows : 0)), gh, xp, xs, live);
      if (gh.sub == 0 && live) s_act[P] = silu(gu.x) * gu.y;
    }
    if (kDownLate && m0 == 0) issue_down();
    lds_sync();
    if (m0 == 0) Q4MOE_STAMP(3, __builtin_amdgcn_s_memrealtime());
    if (nm > 0) publish_units(p.act, p.act_copy_words, I, s_act, nm, epoch, [&](int m) { return unit_of(m0 + m); });
    if (m0 == 0 && has_shared && sh_units > 0)
      publish_units(p.act, p.act_copy_words, I, s_sh, min(sh_units, nbatch_units), epoch,
                    [&](int m) { return make_int2(k, (b + m * NB) * kUnitRows); });
    lds_sync();  // s_act is reused
  }
  // (rarely: more shared units than one batch holds, i.e. fewer than I / 256 workgroups)
  for (int m0 = nbatch_units; m0 < sh_units; m0 += nbatch_units) {
    const int nm = min(nbatch_units, sh_units - m0);
    if constexpr (kQ8Shared) {
      for (int m = wv; m < nm; m += kWaves) {
        const float2 gu = unit_gate_up_q8(L, (b + (m0 + m) * NB) * kUnitRows, xf);
        if ((lane & 7) == 0) s_sh[m * kUnitRows + (lane >> 3)] = silu(gu.x) * gu.y;
      }
    } else {
      const int np = nm * kUnitRows;
      for (int q = 0; q * PS < np; ++q) {
        const int P = q * PS + wv * gh.RPW + gh.lg;
        const bool live = P < np;
        const int i = live ? (b + (m0 + P / kUnitRows) * NB) * kUnitRows + P % kUnitRows : 0;
        const float2 gu = pair_dot_now(shared_pair_ref(L, i), gh, xp, xs, live);
        if (gh.sub == 0 && live) s_sh[P] = silu(gu.x) * gu.y;
      }
    }
    lds_sync();
    publish_units(p.act, p.act_copy_words, I, s_sh, nm, epoch, [&](int m) { return make_int2(k, (b + (m0 + m) * NB) * kUnitRows); });
    lds_sync();
  }

  // ================================================================ phase C
  // routed slots and the shared slot (an 8-bit shared expert's slot also as fp32 into af)
  stage_tagged_split(p.act + (size_t)(b % kCopies) * p.act_copy_words, nslot, I, ap, as, epoch, timeouts,
                     kQ8Shared && !kFast ? af : nullptr, k * I);
  lds_sync();  // activations staged
  Q4MOE_STAMP(4, __builtin_amdgcn_s_memrealtime());
  {
    constexpr int ST = chunk_stride<2>();
    // fast form: a routed task's part from its row chunk
    auto routed_part = [&](const DnRegs& d, int q) {
      const int task = q * PSd + wv * gd.RPW + gd.lg;
      const bool live = task < dtasks_r;
      const int j = live ? task / kOutRows : 0, c = gd.sub;
      float part = affine_term(chunk_pdot<2>(d.c, ap + ((size_t)j * CI + c) * ST), as[j * CI + c], d.s, d.bb);
      part = group_sum_rt(part, gd.lr);
      if (gd.sub == 0 && live) s_red[j * kOutRows + task % kOutRows] = part;
    };
    // fast form: shared row rb * 8 + wv, lane l on columns 8l .. 8l + 7 (block l % 4 of
    // chunk l / 4); the group's bias term is added once, by its first lane
    auto shared_part = [&](const ShDnRegs& d) {
      const int c = lane >> 2, g = lane >> 3;
      const uint32_t* hv = ap + ((size_t)k * CI + c) * ST + 4 * (lane & 3);
      const uint4 hi = *reinterpret_cast<const uint4*>(hv), lo = *reinterpret_cast<const uint4*>(hv + 16);
      uint32_t pr[4];
      if constexpr (kQ8Shared) {
        q8_block_pairs(d.c.x, d.c.y, pr);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = nib_pair(d.c.x, 4 * i);
      }
      float p0 = dot2_bf16(pr[0], hi.x, 0.f), p1 = dot2_bf16(pr[1], hi.y, 0.f);
      p0 = dot2_bf16(pr[2], hi.z, p0);
      p1 = dot2_bf16(pr[3], hi.w, p1);
      p0 = dot2_bf16(pr[0], lo.x, p0);
      p1 = dot2_bf16(pr[1], lo.y, p1);
      p0 = dot2_bf16(pr[2], lo.z, p0);
      p1 = dot2_bf16(pr[3], lo.w, p1);
      const float sc = bf16_bits_to_f32(d.s), bi = bf16_bits_to_f32(d.bb);
      // 8-bit: codes are q; 4-bit: codes are 128 + q (bias - 128 * scale is exact)
      const float cb = kQ8Shared ? bi : bi - 128.0f * sc;
      const float gsum = (lane & 7) == 0 ? as[k * CI + 2 * g] + as[k * CI + 2 * g + 1] : 0.f;
      const float part = group_sum_rt(fmaf(sc, p0 + p1, cb * gsum), 6);
      if (lane == 0) s_red[k * kOutRows + wv] = part;
    };
    for (int rb = b; rb < nblocks; rb += NB) {
      if constexpr (kFast) {
        const bool first = rb == b;
#pragma unroll
        for (int q = 0; q < kDnSlots; ++q) {
          if (q < dpasses_r) {
            if (first && q < dn_pfp) {
              routed_part(dnr[q], q);
            } else {
              DnRegs d;
              load_dn(q, rb, d);
              routed_part(d, q);
            }
          }
        }
        for (int q = kDnSlots; q < dpasses_r; ++q) {  // (more passes than prefetched: loaded now)
          DnRegs d;
          load_dn(q, rb, d);
          routed_part(d, q);
        }
        if (has_shared) {
          if (first) {
            shared_part(shdn);
          } else {
            ShDnRegs d;
            load_shdn(rb, d);
            shared_part(d);
          }
        }
      } else {
        for (int q = 0; q < dpasses; ++q) {
          const int task = q * PSd + wv * gd.RPW + gd.lg;
          const bool live = task < dtasks;
          const int2 jr = task_jr(task);
          const int j = live ? jr.x : 0, n = rb * kOutRows + jr.y;
          float part = 0.f;
          if (kQ8Shared && j == k) {
            part = q8_down_row(L, n, af, gd.sub, gd.LR, gd.lr, live);
          } else {
            if (live) {
              const uint4* cr;
              const uint16_t *sr, *br;
              down_row(j, n, cr, sr, br);
              for (int c = gd.sub; c < CI; c += gd.LR)
                part += affine_term(chunk_pdot<2>(cr[c], ap + ((size_t)j * CI + c) * ST), as[j * CI + c], sr[c >> 1],
                                    br[c >> 1]);
            }
            part = group_sum_rt(part, gd.lr);
          }
          if (gd.sub == 0 && live) s_red[j * kOutRows + jr.y] = part;
        }
      }
      lds_sync();
      if (t < kOutRows) {
        const int n = rb * kOutRows + t;
        float acc = 0.f;
        for (int j = 0; j < nslot; ++j) acc = fmaf(s_w[j], s_red[j * kOutRows + t], acc);  // fixed slot order
        if (p.out_mode == kOutBf16Residual) acc += bf16_bits_to_f32(p.x[n]);
        if (p.out_mode != kOutF32)
          reinterpret_cast<uint16_t*>(p.y)[n] = (uint16_t)f32_to_bf16_bits(acc);
        else
          reinterpret_cast<float*>(p.y)[n] = acc;
      }
      lds_sync();  // s_red is reused
    }
  }
  Q4MOE_STAMP(5, __builtin_amdgcn_s_memrealtime());
}

#define Q4MOE_DECODE_KERNEL(name, q8r, gated, q8sh)                                                  \
  __global__ __launch_bounds__(kThreads) void name(DecodeParams p) { decode_layer<q8r, gated, q8sh, true>(p); } \
  __global__ __launch_bounds__(kThreads) void name##_any(DecodeParams p) { decode_layer<q8r, gated, q8sh, false>(p); }
Q4MOE_DECODE_KERNEL(decode_layer_kernel, false, false, false)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_kernel, true, false, false)
Q4MOE_DECODE_KERNEL(decode_layer_gated_kernel, false, true, false)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_gated_kernel, true, true, false)
Q4MOE_DECODE_KERNEL(decode_layer_q8shared_kernel, false, false, true)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_q8shared_kernel, true, false, true)
Q4MOE_DECODE_KERNEL(decode_layer_gated_q8shared_kernel, false, true, true)
Q4MOE_DECODE_KERNEL(decode_layer_q8router_gated_q8shared_kernel, true, true, true)
#undef Q4MOE_DECODE_KERNEL

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t decode_lds(const DecodeLayer& L) {
  const int nslot = L.top_k + (L.has_shared ? 1 : 0);
  size_t b = (size_t)(L.hidden >> 5) * (chunk_stride<1>() * 4 + 4) +
             (size_t)nslot * (L.inter >> 5) * (chunk_stride<2>() * 4 + 4);
  if (L.has_shared && L.sh_q8) b += 16 + (size_t)((L.hidden >> 6) + (L.inter >> 6)) * kQ8Pad * 4;
  return b;
}

typedef void (*DecodeKernel)(DecodeParams);

DecodeKernel decode_kernel_for(const DecodeLayer& L) {
  static const DecodeKernel kernels[2][2][2][2] = {
      {{{decode_layer_kernel_any, decode_layer_q8shared_kernel_any},
        {decode_layer_gated_kernel_any, decode_layer_gated_q8shared_kernel_any}},
       {{decode_layer_q8router_kernel_any, decode_layer_q8router_q8shared_kernel_any},
        {decode_layer_q8router_gated_kernel_any, decode_layer_q8router_gated_q8shared_kernel_any}}},
      {{{decode_layer_kernel, decode_layer_q8shared_kernel},
        {decode_layer_gated_kernel, decode_layer_gated_q8shared_kernel}},
       {{decode_layer_q8router_kernel, decode_layer_q8router_q8shared_kernel},
        {decode_layer_q8router_gated_kernel, decode_layer_q8router_gated_q8shared_kernel}}}};
  const int q8 = L.router_q8.codes != nullptr, gated = L.sh_gate_w != nullptr && L.has_shared,
            q8sh = L.has_shared && L.sh_q8;
  // the fast form: the compiled shape (one 16-byte word of every gate/up and down row per
  // lane, one word of a router row per thread)
  const int fast = L.hidden == kFastHidden && L.inter == kFastInter;
  return kernels[fast][q8][gated][q8sh];
}

int decode_grid() {
  int blocks = device_cu_count();
  return blocks > kMaxBlocks ? kMaxBlocks : blocks;
}

}  // namespace

// bytes between the copies of the tagged activations: the copy rounded up to 4 KB plus
// 256 bytes, so that consecutive copies start on different channels
size_t act_copy_bytes(int top_k, int inter) { return (((size_t)(top_k + 1) * inter * 8 + 4095) & ~size_t(4095)) + 256; }

size_t decode_workspace_bytes(int hidden, int inter, int n_experts, int top_k) {
  (void)hidden;
  (void)n_experts;
  return align256(sizeof(DecodeWs)) + (size_t)kCopies * act_copy_bytes(top_k, inter);
}

size_t decode_lds_bytes(const DecodeLayer& L) { return decode_lds(L); }

// Every workgroup of the grid waits on words that the others publish, so all of them
// must be resident at once: one workgroup per CU must fit (registers and LDS).  The
// answer is cached per device and LDS size.
bool decode_fits(const DecodeLayer& L) {
  struct Entry {
    int dev;
    DecodeKernel k;
    size_t lds;
    bool ok;
  };
  static Entry cache[32];
  static int ncache = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const DecodeKernel kern = decode_kernel_for(L);
  const size_t lds = decode_lds(L);
  for (int i = 0; i < ncache; ++i)
    if (cache[i].dev == dev && cache[i].k == kern && cache[i].lds == lds) return cache[i].ok;
  int per_cu = 0;
  const bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kThreads,
                                                               lds) == hipSuccess &&
                  per_cu >= 1;
  if (ncache < 32) cache[ncache++] = Entry{dev, kern, lds, ok};
  return ok;
}

// ---- the no-allocation form: the workspace is a file-scope device array.
// Each device that runs the library holds its own copy of `scratch` until the process
// ends; host code uses the per-device address from hipGetSymbolAddress (the array's
// name in host code is only a stand-in).  The array starts as zeros, which is the state
// the decode workspace needs before its first use; every call leaves it ready for the
// next one.  Calls on one device share it, so calls that overlap on one device race.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

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
  p.act_copy_words = (int64_t)act_copy_bytes(L.top_k, L.inter) / 8;
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(decode_kernel_for(L)), dim3(decode_grid()),
                                       dim3(kThreads), args, decode_lds(L), stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace q4moe

#ifdef Q4MOE_DECODE_STAMPS
// Diagnostic build only (not part of the library's interface): copies the stamp array
// ([4][1024][8] uint64, slot epoch % 4, stamps as listed above) to host memory.
extern "C" int q4moe_decode_stamps(void* host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(q4moe::g_decode_stamps), bytes);
}
#endif
