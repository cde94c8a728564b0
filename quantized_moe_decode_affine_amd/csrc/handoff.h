// Handoffs between the workgroups of one co-resident grid (the decode launches).
//
// A value handed from one workgroup to another is one aligned 64-bit word
// {epoch:hi32, fp32 bits:lo32} written by one store of the launch, so a
// consumer's device-coherent load both reads the value and tells whether it is
// there yet (single-copy atomicity of the 64-bit store; no ordering between two
// locations is needed).  The epoch of a launch is agreed through per-group
// arrival counters at the head of the workspace: each workgroup adds one to
// its group's counter and takes (epoch field + 1); the last arrival of a group
// resets the count and advances the epoch field, so every workgroup of the
// next launch (stream-ordered after this one) takes the next value.  Every
// poll is bounded: a value that never arrives is counted in `timeouts` (byte
// 2048 of the workspace, read by the host) and leaves a wrong result, never a
// hang.
#pragma once

#include <stddef.h>

#include "common.h"
#include "topk.h"

namespace q4moe {

constexpr int kEpochGroups = 8;
constexpr unsigned kPollLimit = 1u << 18;  // ~0.25 s of polling

struct HandoffHead {
  unsigned long long group_ctr[kEpochGroups][32];  // {epoch:hi32, arrivals:lo32}, one 256-byte slot each
  unsigned timeouts;
  unsigned pad[63];
};
static_assert(offsetof(HandoffHead, timeouts) == 2048, "the host reads the timeout count at byte 2048");

__device__ __forceinline__ unsigned long long tag_word(uint32_t epoch, float v) {
  return ((unsigned long long)epoch << 32) | __float_as_uint(v);
}

// Arrival of workgroup b of NB (one thread): returns the counter's previous value.
__device__ __forceinline__ unsigned long long epoch_arrive(HandoffHead* h, int b) {
  return __hip_atomic_fetch_add(&h->group_ctr[b % kEpochGroups][0], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The launch's epoch from an arrival's previous value (the same thread); the group's
// last arrival resets the count and advances the epoch field.
__device__ __forceinline__ uint32_t epoch_finish(HandoffHead* h, int b, int NB, unsigned long long old) {
  const int eg = b % kEpochGroups;
  const unsigned egsize = (NB - eg + kEpochGroups - 1) / kEpochGroups;
  if ((uint32_t)old == egsize - 1)
    __hip_atomic_fetch_add(&h->group_ctr[eg][0], (1ull << 32) - egsize, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (uint32_t)(old >> 32) + 1u;
}

// Top-k of E logits by one wave, polling the epoch-tagged words that other
// workgroups publish (word e * kStride) until every one carries `epoch` (bounded;
// a timeout is counted).  Lane l holds ids [l*V, l*V + V) (wave_topk_keys: equal
// logits resolve to the lower expert id).  Writes ids/weights (renormalised softmax
// of the kept logits) to LDS and, when given, to ids_out/w_out.
template <int V, int kStride>
__device__ __forceinline__ void wave_topk_tagged(const unsigned long long* tags, int E, int k, uint32_t epoch,
                                                 unsigned* timeouts, int32_t* s_ids, float* s_w, int32_t* ids_out,
                                                 float* w_out) {
  const int lane = lane_id();
  uint32_t key[V];
  int id[V];
#pragma unroll
  for (int j = 0; j < V; ++j) id[j] = lane * V + j;
  // device-coherent 8-byte loads, one per logit slot; slots past E read as zeros (bounds check)
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned long long*>(tags), 0, E * kStride * 8, kBufferRsrcWord3);
  for (unsigned spins = 0;; ++spins) {
    bool ready = true;
    uint2 t[V];
#pragma unroll
    for (int j = 0; j < V; ++j)  // all loads in flight together
      t[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, id[j] * kStride * 8, 0,
                                                                         kLoadDeviceScope));
#pragma unroll
    for (int j = 0; j < V; ++j) {
      key[j] = t[j].x;
      ready &= id[j] >= E || t[j].y == epoch;
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

}  // namespace q4moe
