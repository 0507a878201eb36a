// Top-k routing of one token by one wavefront, shared by the router kernel
// and the fused decode layer.  The routable subset is the kept set of the
// DGX Spark page ("The numbers"); ranking is (logit descending, expert index
// ascending); weights are the softmax of the k selected logits.
#pragma once

#include "common.cuh"

namespace moe {

// Selection key: routable class, then logit, then lower expert index, packed
// so that a larger unsigned key is the better candidate:
//   bits 42-43 class (2 routable, 1 not routable, 0 absent or taken),
//   bits 10-41 the logit mapped to an order-preserving unsigned integer
//              (-0 folded onto +0, NaN read as -inf),
//   bits  0-9  1023 - expert.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  if (v != v) v = -INFINITY;
  v += 0.0f;  // -0 -> +0
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

struct RoutePick {
  int expert;    // expert of slot `lane` (lanes < k)
  float weight;  // its routing weight
  int routable;  // 1 if the expert is in the routable subset
};

// Every lane of the wavefront calls this; lane j < k receives slot j.
template <int NPL>
__device__ __forceinline__ RoutePick route_token(const float* __restrict__ row, int E, int k,
                                                 const int32_t* __restrict__ e2s, int lane) {
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const uint64_t cls = (e2s == nullptr || e2s[e] >= 0) ? 2 : 1;
      key[i] = (cls << 42) | ((uint64_t)ordered_bits(row[e]) << 10) | (uint64_t)(1023 - e);
    } else {
      key[i] = 0;
    }
  }
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) best = umax64(best, key[i]);
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (key[i] == best) key[i] = 0;  // keys are unique: only the winner matches
    if (lane == j) mine = best;
  }
  const int cls = (int)(mine >> 42);
  const int e = 1023 - (int)(mine & 1023u);
  const float v = from_ordered_bits((uint32_t)(mine >> 10));
  const float v0 = __shfl(v, 0, 64);
  float d = v - v0;
  if (d != d) d = 0.0f;
  const float ex = (lane < k && cls == 2) ? expf(d) : 0.0f;
  const float s = wave_sum_dpp(ex);
  RoutePick r;
  r.expert = (cls > 0 && e < E) ? e : 0;
  r.weight = s > 0.0f ? ex / s : 0.0f;
  r.routable = cls == 2;
  return r;
}

}  // namespace moe
