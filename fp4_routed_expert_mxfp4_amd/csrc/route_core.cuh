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

// General form (any number of routable experts): k rounds of a 64-bit wave
// max over every lane's candidates.  Every lane calls this; lane j < k
// receives slot j.
template <int NPL>
__device__ __forceinline__ RoutePick route_token_keys64(const float* __restrict__ row, int E, int k,
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
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
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

// Every lane gets the maximum over all 64 lanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppXor1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppXor2, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppHalfMirror, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppMirror, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)b[0], (uint32_t)b[1]);
}

// The same selection when at least k experts are routable (the documented
// precondition; otherwise route_token_keys64 runs): then every pick is
// routable, so a candidate is its order-preserving 32-bit logit (0 for a
// non-routable or absent one, below every routable value) and its expert
// index.  Each lane sorts its candidates once by (logit descending, expert
// ascending); a round is then one 32-bit wave max over the lanes' heads, a
// ballot for ties (rare: the lowest expert index among the tied heads wins),
// and the winning lane pops its head.  The picks, their order and the
// weights are exactly those of route_token_keys64.
template <int NPL>
__device__ __forceinline__ RoutePick route_token(const float* __restrict__ row, int E, int k,
                                                 const int32_t* __restrict__ e2s, int lane) {
  uint64_t key[NPL];  // (ordered logit << 32) | (0xFFFF - expert); 0 = no candidate
  int nrout = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    const bool ok = e < E && (e2s == nullptr || e2s[e] >= 0);
    key[i] = ok ? ((uint64_t)ordered_bits(row[e]) << 32) | (uint64_t)(0xFFFFu - (uint32_t)e) : 0;
    nrout += __builtin_popcountll(__ballot(ok));
  }
  if (nrout < k) return route_token_keys64<NPL>(row, E, k, e2s, lane);
  // sort descending (keys are unique, so the order is total): odd-even transposition
#pragma unroll
  for (int p = 0; p < NPL; ++p)
#pragma unroll
    for (int i = p & 1; i + 1 < NPL; i += 2) {
      const uint64_t a = key[i], b = key[i + 1];
      key[i] = a > b ? a : b;
      key[i + 1] = a > b ? b : a;
    }
  uint32_t mine_v = 0, mine_e = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hv = (uint32_t)(key[0] >> 32), hl = (uint32_t)key[0];
    const uint32_t best = wave_max_u32(hv);
    uint64_t tied = __ballot(hv == best);
    if (__builtin_popcountll(tied) > 1) {  // equal logits: the lowest expert index, i.e. the largest low word
      const uint32_t bl = wave_max_u32(hv == best ? hl : 0u);
      tied = __ballot(hv == best && hl == bl);
    }
    const int wl = __builtin_ctzll(tied);
    const uint32_t e = 0xFFFFu - (uint32_t)__builtin_amdgcn_readlane((int)hl, wl);
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i + 1 < NPL; ++i) key[i] = key[i + 1];
      key[NPL - 1] = 0;
    }
    if (lane == j) {
      mine_v = best;
      mine_e = e;
    }
  }
  const float v = from_ordered_bits(mine_v);
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float d = v - v0;
  if (d != d) d = 0.0f;
  const float ex = lane < k ? expf(d) : 0.0f;
  const float s = wave_sum_dpp(ex);
  RoutePick r;
  r.expert = lane < k ? (int)mine_e : 0;
  r.weight = s > 0.0f ? ex / s : 0.0f;
  r.routable = lane < k;
  return r;
}

}  // namespace moe
