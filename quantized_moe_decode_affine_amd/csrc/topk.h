// Wave-level top-k selection over a logit vector (router softmax -> top-k ->
// renormalise; lily README, introduction: a 35B-A3B mixture-of-experts model
// whose router picks the active experts).
#pragma once

#include "common.h"

namespace q4moe {

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;

// Top-k of the logit vector by one wave: k rounds of a wave-wide maximum of
// order-preserving keys; equal logits resolve to the lower expert id because
// each lane holds a contiguous block of ids and the lowest matching lane wins.
__device__ inline void wave_topk(const float* logits, int E, int k, int32_t* ids, float* w) {
  const int lane = lane_id();
  constexpr int V = kMaxExperts / kWave;
  const int per = (E + kWave - 1) / kWave;
  uint32_t key[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane * per + j;
    key[j] = (j < per && e < E) ? float_key(logits[e]) : 0u;
  }
  float top = 0.f, sum = 0.f, my_ex = 0.f;
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t lb = 0;
    int lj = 0;
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (key[j] > lb) { lb = key[j]; lj = j; }
    uint32_t m = lb;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, kWave));
    const unsigned long long hit = __ballot(lb == m);
    const int src = __ffsll((long long)hit) - 1;
    const int id = __shfl(lane * per + lj, src, kWave);
    if (lane == src) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (j == lj) key[j] = 0u;
    }
    const float val = logits[id];
    if (r == 0) top = val;
    const float ex = expf(val - top);
    sum += ex;
    if (lane == r) { my_id = id; my_ex = ex; }
  }
  if (lane < k) { ids[lane] = my_id; w[lane] = my_ex / sum; }
}

}  // namespace q4moe
