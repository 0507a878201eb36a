// Top-k router and token-to-expert bucketing (gfx950).
//
// Router: one wavefront per token; each lane keeps its share of the token's
// logits in registers and k rounds of a wave-wide arg-max pick the experts in
// rank order (logit descending, expert index ascending -- the tie rule makes
// the selection a total order, so the butterfly reduction is deterministic).
// The weights are the softmax of the k selected logits.  The routable subset
// follows the DGX Spark page ("The numbers": only a kept subset of experts is
// routable).
//
// Bucketing: the (token, slot) rows of the argonautlabs report ("30 September
// follow-up") sorted stably by expert.  One workgroup of 1024 threads builds
// the histogram, the exclusive scan and then scatters the pairs in rounds of
// 1024; inside a round each wavefront ranks equal experts with ballots and the
// per-wave histograms give the offset of earlier waves, so the order is the
// stable (expert, pair) order without any atomic-order dependence.
#include "common.cuh"
#include "kernels.h"

namespace moe {

namespace {

struct Pick {
  int cls;   // 2 routable, 1 not routable, 0 absent / already taken
  float v;
  int e;
};

__device__ __forceinline__ bool better(const Pick& a, const Pick& b) {
  if (a.cls != b.cls) return a.cls > b.cls;
  if (a.v != b.v) return a.v > b.v;
  return a.e < b.e;
}

template <int NPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, const int32_t* __restrict__ e2s,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront leaves together
  const float* row = logits + (size_t)t * E;
  float v[NPL];
  int cls[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      float x = row[e];
      v[i] = (x != x) ? -INFINITY : x;
      cls[i] = (e2s == nullptr || e2s[e] >= 0) ? 2 : 1;
    } else {
      v[i] = -INFINITY;
      cls[i] = 0;
    }
  }
  Pick mine{0, -INFINITY, 0x7FFFFFFF};  // lane j keeps pick j
  for (int j = 0; j < k; ++j) {
    Pick best{0, -INFINITY, 0x7FFFFFFF};
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      Pick c{cls[i], v[i], lane + 64 * i};
      if (c.cls > 0 && better(c, best)) best = c;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      Pick o{__shfl_xor(best.cls, off, 64), __shfl_xor(best.v, off, 64), __shfl_xor(best.e, off, 64)};
      if (better(o, best)) best = o;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i == best.e) cls[i] = 0;
    if (lane == j) mine = best;
  }
  const float v0 = __shfl(mine.v, 0, 64);
  float d = mine.v - v0;
  if (d != d) d = 0.0f;
  const float ex = (lane < k && mine.cls == 2) ? expf(d) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = mine.e < E ? mine.e : 0;
    w[(size_t)t * k + lane] = s > 0.0f ? ex / s : 0.0f;
  }
}

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int P,
                                                               int E, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pair,
                                                               int32_t* __restrict__ pair_to_row) {
  __shared__ int cursor[kMaxExperts];
  __shared__ int hist[kPermWaves][kMaxExperts];
  __shared__ int wave_tot[kPermWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < kMaxExperts; e += kPermThreads) {
    cursor[e] = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) hist[w][e] = 0;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kPermThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cursor[e], 1);
  }
  __syncthreads();

  // exclusive scan of the counts (E <= 1024: one expert per thread)
  const int c = tid < E ? cursor[tid] : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const int excl = before + incl - c;
  if (tid < E) {
    offsets[tid] = excl;
    cursor[tid] = excl;
    if (tid == E - 1) offsets[E] = excl + c;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < P; base += kPermThreads) {
    const int p = base + tid;
    const int e = p < P ? ids[p] : -1;
    const bool valid = (e >= 0 && e < E);
    if (p < P && !valid) pair_to_row[p] = -1;
    uint64_t active = __ballot(valid);
    int my_rank = 0, my_cnt = 0;
    bool leader = false;
    while (active) {
      const int ll = __ffsll((unsigned long long)active) - 1;
      const int ev = __shfl(e, ll, 64);
      const bool match = valid && e == ev;
      const uint64_t m = __ballot(match);
      if (match) {
        my_rank = __popcll(m & lt_mask);
        my_cnt = __popcll(m);
        leader = (lane == ll);
      }
      active &= ~m;
    }
    if (leader) hist[wave][e] = my_cnt;
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += hist[w][e];
      const int pos = cursor[e] + pre + my_rank;
      sorted_pair[pos] = p;
      pair_to_row[p] = pos;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&cursor[e], my_cnt);
      hist[wave][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, const int32_t* e2s, int32_t* ids,
                        float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  const int npl = (E + 63) / 64;
  if (npl <= 1)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, T, E, k, e2s, ids, w);
  else if (npl <= 2)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, T, E, k, e2s, ids, w);
  else if (npl <= 4)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, T, E, k, e2s, ids, w);
  else if (npl <= 8)
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, T, E, k, e2s, ids, w);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, logits, T, E, k, e2s, ids, w);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_to_row, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, P, E, offsets,
                     sorted_pair, pair_to_row);
  return hipGetLastError();
}

}  // namespace moe
