// Wave-level top-k over a logit vector: softmax over all experts, keep the k
// largest, renormalise their probabilities (lily README, introduction: a
// 35B-A3B mixture-of-experts model whose router picks the active experts).
//
// k rounds of a wave-wide maximum of order-preserving keys (DPP and permlane
// steps, no LDS traffic).  Each lane holds a contiguous block of expert ids,
// so among equal logits the lowest lane, hence the lowest expert id, wins.
// Softmax over all experts followed by renormalisation over the kept ones is
// the softmax of the kept logits, which is what is computed.
#pragma once

#include "common.h"

namespace q4moe {

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;

// Writes ids[0..k) (descending logit) and w[0..k) (renormalised weights); lanes < k write.
// COHERENT: read the logits with agent-scope loads (they were written by other
// workgroups of the same grid).
template <bool COHERENT = false>
__device__ inline void wave_topk(const float* logits, int E, int k, int32_t* ids, float* w) {
  const int lane = lane_id();
  constexpr int V = kMaxExperts / kWave;
  const int per = (E + kWave - 1) / kWave;
  uint32_t key[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane * per + j;
    key[j] = (j < per && e < E) ? float_key(COHERENT ? ld_agent(logits + e) : logits[e]) : 0u;
  }
  float top = 0.f, my_val = 0.f;
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t lb = 0;
    int lj = 0;
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (j < per && key[j] > lb) { lb = key[j]; lj = j; }
    const uint32_t m = wave_max_u32(lb);
    const unsigned long long hit = __ballot(lb == m);
    const int src = __builtin_ctzll(hit);
    const int id = __builtin_amdgcn_readlane(lane * per + lj, src);
    if (lane == src) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (j == lj) key[j] = 0u;
    }
    const float val = key_float(m);
    if (r == 0) top = val;
    if (lane == r) { my_id = id; my_val = val; }
  }
  const float ex = lane < k ? expf(my_val - top) : 0.f;
  const float sum = group_sum_rt(ex, 6);
  if (lane < k) {
    ids[lane] = my_id;
    w[lane] = ex / sum;
  }
}

}  // namespace q4moe
