// Batch-1 decode step of one MoE feed-forward layer.
//
// The step is a dependent chain of weight streams (lily-qwen3.8-flash-next
// README, "How the speed was achieved": decode is bandwidth-bound and its
// kernels are tuned against the chain of reads):
//   phase A: router logits (bf16 GEMV) and the shared expert's gate/up rows,
//            which do not depend on the routing;
//   phase B: top-k of the logits (recomputed in every workgroup from the
//            1 KB logit vector, so no extra pass is needed) and the routed
//            experts' gate/up rows, SwiGLU fused: a = silu(g) * u in fp32;
//   phase C: the down rows of all selected experts plus the shared expert for
//            each output row, weighted and summed in registers (no atomics,
//            a fixed summation order), y written once.
// Intermediates (logits, a, routing) live in the caller's workspace.
#include "kernels.h"
#include "topk.h"
#include "vecstage.h"

namespace q4moe {

namespace {

struct DecodeParams {
  DecodeLayer L;
  const uint16_t* x;  // [H]
  void* y;            // [H]
  int out_bf16;
  int32_t* ids_out;   // nullable [k]
  float* w_out;       // nullable [k]
  float* logits;      // ws [E]
  float* a;           // ws [k+1][I]
  int32_t* sel_ids;   // ws [k]
  float* sel_w;       // ws [k]
  int lsH;            // log2 lanes per row for k = hidden
  int lsI;            // log2 lanes per row for k = inter
};

// Dot of gate row and up row i of one expert against the staged x; every lane
// of the row's lane group returns (g, u).
__device__ __forceinline__ float2 gate_up_dot(const Q4Mat& gm, const Q4Mat& um, int64_t mat_off_codes,
                                              int64_t mat_off_groups, int i, int H, int sub, int L,
                                              const uint32_t* vp, const float* vs) {
  constexpr int ST = chunk_stride<1>();
  const int C = H >> 5, G = H >> 6;
  const uint4* gc = reinterpret_cast<const uint4*>(gm.codes + mat_off_codes) + (int64_t)i * C;
  const uint4* uc = reinterpret_cast<const uint4*>(um.codes + mat_off_codes) + (int64_t)i * C;
  const uint16_t* gs = gm.scales + mat_off_groups + (int64_t)i * G;
  const uint16_t* gb = gm.biases + mat_off_groups + (int64_t)i * G;
  const uint16_t* us = um.scales + mat_off_groups + (int64_t)i * G;
  const uint16_t* ub = um.biases + mat_off_groups + (int64_t)i * G;
  float ag = 0.f, au = 0.f;
  for (int g = sub; g < G; g += L) {
    const uint4 g0 = gc[2 * g], g1 = gc[2 * g + 1];
    const uint4 u0 = uc[2 * g], u1 = uc[2 * g + 1];
    const uint32_t gsb = gs[g], gbb = gb[g], usb = us[g], ubb = ub[g];
    const uint32_t* v = vp + 2 * g * ST;
    const float vsum = vs[2 * g] + vs[2 * g + 1];
    ag += affine_term(chunk_pdot<1>(g0, v) + chunk_pdot<1>(g1, v + ST), vsum, gsb, gbb);
    au += affine_term(chunk_pdot<1>(u0, v) + chunk_pdot<1>(u1, v + ST), vsum, usb, ubb);
  }
  for (int m = 1; m < L; m <<= 1) {
    ag += __shfl_xor(ag, m, kWave);
    au += __shfl_xor(au, m, kWave);
  }
  return make_float2(ag, au);
}

__global__ __launch_bounds__(256) void decode_phase_a(DecodeParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  const int H = p.L.hidden, I = p.L.inter, E = p.L.n_experts;
  const int C = H >> 5;
  uint32_t* vp = smem;
  float* vs = reinterpret_cast<float*>(smem + C * chunk_stride<1>());
  if (p.L.has_shared) {
    stage_bf16_vector(p.x, C, vp, vs);
    __syncthreads();
  }
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  const int wave = blockIdx.x * wpb + threadIdx.x / kWave;
  const int nwaves = gridDim.x * wpb;
  const int L = 1 << p.lsH, sub = lane & (L - 1), rsub = lane >> p.lsH, rpi = kWave >> p.lsH;
  const int pair_items = p.L.has_shared ? (I + rpi - 1) / rpi : 0;
  const int items = E + pair_items;
  for (int it = wave; it < items; it += nwaves) {
    if (it < E) {
      // router row `it`: bf16 . bf16, natural pair order on both sides
      const uint4* r = reinterpret_cast<const uint4*>(p.L.router + (size_t)it * H);
      const uint4* xv = reinterpret_cast<const uint4*>(p.x);
      float acc0 = 0.f, acc1 = 0.f;
      for (int c = lane; c < (H >> 3); c += kWave) {
        const uint4 w = r[c], v = xv[c];
        acc0 = dot2_bf16(w.x, v.x, acc0);
        acc1 = dot2_bf16(w.y, v.y, acc1);
        acc0 = dot2_bf16(w.z, v.z, acc0);
        acc1 = dot2_bf16(w.w, v.w, acc1);
      }
      float acc = group_sum<kWave>(acc0 + acc1);
      if (lane == 0) p.logits[it] = acc;
    } else {
      const int i = (it - E) * rpi + rsub;
      if (i < I) {
        float2 gu = gate_up_dot(p.L.sh_gate, p.L.sh_up, 0, 0, i, H, sub, L, vp, vs);
        if (sub == 0) p.a[(size_t)p.L.top_k * I + i] = silu(gu.x) * gu.y;
      }
    }
  }
}

__global__ __launch_bounds__(256) void decode_phase_b(DecodeParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ int32_t s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int H = p.L.hidden, I = p.L.inter, k = p.L.top_k;
  const int C = H >> 5;
  uint32_t* vp = smem;
  float* vs = reinterpret_cast<float*>(smem + C * chunk_stride<1>());
  if (threadIdx.x < kWave) {
    wave_topk(p.logits, p.L.n_experts, k, s_ids, s_w);
    if (blockIdx.x == 0 && threadIdx.x < k) {
      p.sel_ids[threadIdx.x] = s_ids[threadIdx.x];
      p.sel_w[threadIdx.x] = s_w[threadIdx.x];
      if (p.ids_out) p.ids_out[threadIdx.x] = s_ids[threadIdx.x];
      if (p.w_out) p.w_out[threadIdx.x] = s_w[threadIdx.x];
    }
  }
  stage_bf16_vector(p.x, C, vp, vs);
  __syncthreads();

  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  const int wave = blockIdx.x * wpb + threadIdx.x / kWave;
  const int nwaves = gridDim.x * wpb;
  const int L = 1 << p.lsH, sub = lane & (L - 1), rsub = lane >> p.lsH, rpi = kWave >> p.lsH;
  const int per_slot = (I + rpi - 1) / rpi;
  const int64_t mat_codes = (int64_t)I * (H >> 3), mat_groups = (int64_t)I * (H >> 6);
  for (int it = wave; it < k * per_slot; it += nwaves) {
    const int j = it / per_slot;
    const int i = (it - j * per_slot) * rpi + rsub;
    if (i >= I) continue;
    const int64_t e = s_ids[j];
    float2 gu = gate_up_dot(p.L.gate, p.L.up, e * mat_codes, e * mat_groups, i, H, sub, L, vp, vs);
    if (sub == 0) p.a[(size_t)j * I + i] = silu(gu.x) * gu.y;
  }
}

__global__ __launch_bounds__(128) void decode_phase_c(DecodeParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ int32_t s_ids[kMaxTopK + 1];
  __shared__ float s_w[kMaxTopK + 1];
  constexpr int ST = chunk_stride<2>();
  const int H = p.L.hidden, I = p.L.inter, k = p.L.top_k;
  const int nslot = k + (p.L.has_shared ? 1 : 0);
  const int C = I >> 5, G = I >> 6;
  uint32_t* vp = smem;                                            // [nslot][C][ST]
  float* vs = reinterpret_cast<float*>(smem + (size_t)nslot * C * ST);  // [nslot][C]
  if (threadIdx.x < k) { s_ids[threadIdx.x] = p.sel_ids[threadIdx.x]; s_w[threadIdx.x] = p.sel_w[threadIdx.x]; }
  if (threadIdx.x == 0 && p.L.has_shared) { s_ids[k] = -1; s_w[k] = 1.0f; }
  for (int j = 0; j < nslot; ++j) stage_f32_split_vector(p.a + (size_t)j * I, C, vp + (size_t)j * C * ST, vs + j * C);
  __syncthreads();

  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  const int wave = blockIdx.x * wpb + threadIdx.x / kWave;
  const int nwaves = gridDim.x * wpb;
  const int L = 1 << p.lsI, sub = lane & (L - 1), rsub = lane >> p.lsI, rpi = kWave >> p.lsI;
  const int64_t mat_codes = (int64_t)H * (I >> 3), mat_groups = (int64_t)H * G;
  for (int it = wave; it * rpi < H; it += nwaves) {
    const int n = it * rpi + rsub;
    float acc = 0.f;
    if (n < H) {
      for (int j = 0; j < nslot; ++j) {
        const int e = s_ids[j];
        const Q4Mat& m = e >= 0 ? p.L.down : p.L.sh_down;
        const int64_t oc = e >= 0 ? e * mat_codes : 0, og = e >= 0 ? e * mat_groups : 0;
        const uint4* cr = reinterpret_cast<const uint4*>(m.codes + oc) + (int64_t)n * C;
        const uint16_t* sr = m.scales + og + (int64_t)n * G;
        const uint16_t* br = m.biases + og + (int64_t)n * G;
        float part = 0.f;
        for (int g = sub; g < G; g += L) {
          const uint4 c0 = cr[2 * g], c1 = cr[2 * g + 1];
          const uint32_t* v = vp + ((size_t)j * C + 2 * g) * ST;
          const float vsum = vs[j * C + 2 * g] + vs[j * C + 2 * g + 1];
          part += affine_term(chunk_pdot<2>(c0, v) + chunk_pdot<2>(c1, v + ST), vsum, sr[g], br[g]);
        }
        acc = fmaf(s_w[j], part, acc);
      }
    }
    for (int m = 1; m < L; m <<= 1) acc += __shfl_xor(acc, m, kWave);
    if (n < H && sub == 0) {
      if (p.out_bf16)
        reinterpret_cast<uint16_t*>(p.y)[n] = (uint16_t)f32_to_bf16_bits(acc);
      else
        reinterpret_cast<float*>(p.y)[n] = acc;
    }
  }
}

int lanes_log2(int groups) {
  int r = 0;
  while (r < 6 && (2 << r) <= groups) ++r;
  return r;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

size_t decode_workspace_bytes(int hidden, int inter, int n_experts, int top_k) {
  (void)hidden;
  return align256((size_t)kMaxExperts * 4) + align256((size_t)(top_k + 1) * inter * 4) + align256(kMaxTopK * 4) * 2;
}

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
  p.logits = reinterpret_cast<float*>(w);
  w += align256((size_t)kMaxExperts * 4);
  p.a = reinterpret_cast<float*>(w);
  w += align256((size_t)(L.top_k + 1) * L.inter * 4);
  p.sel_ids = reinterpret_cast<int32_t*>(w);
  w += align256(kMaxTopK * 4);
  p.sel_w = reinterpret_cast<float*>(w);
  p.lsH = lanes_log2(L.hidden / kGroup);
  p.lsI = lanes_log2(L.inter / kGroup);

  const int rpiH = kWave >> p.lsH, rpiI = kWave >> p.lsI;
  const size_t ldsH = (size_t)(L.hidden >> 5) * (chunk_stride<1>() * 4 + 4);
  const int nslot = L.top_k + (L.has_shared ? 1 : 0);
  const size_t ldsI = (size_t)nslot * (L.inter >> 5) * (chunk_stride<2>() * 4 + 4);

  const int items_a = L.n_experts + (L.has_shared ? (L.inter + rpiH - 1) / rpiH : 0);
  hipLaunchKernelGGL(decode_phase_a, dim3((items_a + 3) / 4), dim3(256), ldsH, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items_b = L.top_k * ((L.inter + rpiH - 1) / rpiH);
  hipLaunchKernelGGL(decode_phase_b, dim3((items_b + 3) / 4), dim3(256), ldsH, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items_c = (L.hidden + rpiI - 1) / rpiI;
  hipLaunchKernelGGL(decode_phase_c, dim3((items_c + 1) / 2), dim3(128), ldsI, stream, p);
  return hipGetLastError();
}

}  // namespace q4moe
