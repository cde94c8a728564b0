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

// Top-k of keys held V per lane (order-preserving keys, 0 for no expert; lane l
// holds ids id[0..V), ascending with j and with the lane): each lane sorts its
// keys once, then each of the k rounds is a wave-wide maximum of the lane heads
// and a pop in the winning lane.  Equal keys resolve to the lower id: inside a
// lane by the sort (a swap needs a strictly larger key), across lanes because
// the lowest matching lane wins.  Lanes < k write ids[lane] (descending logit)
// and w[lane] (the renormalised softmax of the kept logits).
template <int V>
__device__ __forceinline__ void wave_topk_keys(uint32_t (&key)[V], int (&id)[V], int k, int32_t* ids, float* w) {
  const int lane = lane_id();
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
    ids[lane] = my_id;
    w[lane] = ex / sum;
  }
}

// wave_topk_keys over E <= 64 * V logits in memory (lane l reads ids l*V .. l*V + V - 1).
template <int V>
__device__ __forceinline__ void wave_topk_sorted(const float* logits, int E, int k, int32_t* ids, float* w) {
  const int lane = lane_id();
  uint32_t key[V];
  int id[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    id[j] = lane * V + j;
    key[j] = id[j] < E ? float_key(logits[id[j]]) : 0u;
  }
  wave_topk_keys<V>(key, id, k, ids, w);
}

}  // namespace q4moe
