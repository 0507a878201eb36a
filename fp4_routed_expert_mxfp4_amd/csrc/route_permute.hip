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
#include "route_core.cuh"

namespace moe {

namespace {

template <int NPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, const int32_t* __restrict__ e2s,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront leaves together
  const RoutePick pick = route_token<NPL>(logits + (size_t)t * E, E, k, e2s, lane);
  if (lane < k) {
    ids[(size_t)t * k + lane] = pick.expert;
    w[(size_t)t * k + lane] = pick.weight;
  }
}

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

struct PermSmem {
  int cursor[kMaxExperts];
  int hist[kPermWaves][kMaxExperts];
  int wave_tot[kPermWaves];
};

__device__ void zero_hist(PermSmem& sm) {
  for (int e = threadIdx.x; e < kMaxExperts; e += kPermThreads) {
    sm.cursor[e] = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) sm.hist[w][e] = 0;
  }
}

// Exclusive scan of c (one value per thread, E <= 1024 threads); returns the
// exclusive prefix of this thread and, in *total, the sum.
__device__ int block_exclusive_scan(PermSmem& sm, int c, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sm.wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kPermWaves; ++w) {
    const int v = sm.wave_tot[w];
    before += w < wave ? v : 0;
    all += v;
  }
  *total = all;
  return before + incl - c;
}

// Stable scatter of the pairs [base, base+1024) given cursor[e] = first row
// of expert e still free.  Within a wavefront equal experts are ranked with
// ballots; the per-wave histograms give the rows taken by earlier wavefronts.
__device__ void scatter_round(PermSmem& sm, const int32_t* __restrict__ ids, int P, int E, int base,
                              int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_row) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
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
  if (leader) sm.hist[wave][e] = my_cnt;
  __syncthreads();
  if (valid) {
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += sm.hist[w][e];
    const int pos = sm.cursor[e] + pre + my_rank;
    sorted_pair[pos] = p;
    pair_to_row[p] = pos;
  }
  __syncthreads();
  if (leader) {
    atomicAdd(&sm.cursor[e], my_cnt);
    sm.hist[wave][e] = 0;
  }
  __syncthreads();
}

// Whole bucketing in one workgroup (used when all pairs fit in one round).
__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pair,
                                                               int32_t* __restrict__ pair_to_row) {
  __shared__ PermSmem sm;
  const int tid = threadIdx.x;
  zero_hist(sm);
  __syncthreads();
  for (int p = tid; p < P; p += kPermThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&sm.cursor[e], 1);
  }
  __syncthreads();
  const int c = tid < E ? sm.cursor[tid] : 0;
  int total;
  const int excl = block_exclusive_scan(sm, c, &total);
  if (tid < E) {
    offsets[tid] = excl;
    sm.cursor[tid] = excl;
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  for (int base = 0; base < P; base += kPermThreads)
    scatter_round(sm, ids, P, E, base, sorted_pair, pair_to_row);
}

// Multi-workgroup bucketing: workgroup b owns pairs [1024b, 1024b+1024).
// (1) per-chunk histograms -> ws[b][e]; (2) one workgroup turns them into the
// first free row of expert e for chunk b and writes the offsets; (3) each
// chunk scatters its pairs from those rows.  The order is the same stable
// (expert, pair) order as the single-workgroup kernel.
__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                     int32_t* __restrict__ ws) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int p = blockIdx.x * kPermThreads + tid;
  if (p < P) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < E) ws[(size_t)blockIdx.x * E + tid] = cnt[tid];
}

__global__ __launch_bounds__(kPermThreads) void permute_scan_kernel(int nchunks, int E, int32_t* __restrict__ ws,
                                                                    int32_t* __restrict__ offsets) {
  __shared__ PermSmem sm;
  const int tid = threadIdx.x;
  int tot = 0;
  if (tid < E)
    for (int b = 0; b < nchunks; ++b) tot += ws[(size_t)b * E + tid];
  int total;
  const int excl = block_exclusive_scan(sm, tid < E ? tot : 0, &total);
  if (tid < E) {
    offsets[tid] = excl;
    int acc = excl;
    for (int b = 0; b < nchunks; ++b) {
      const int t = ws[(size_t)b * E + tid];
      ws[(size_t)b * E + tid] = acc;
      acc += t;
    }
  }
  if (tid == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                       const int32_t* __restrict__ ws,
                                                                       int32_t* __restrict__ sorted_pair,
                                                                       int32_t* __restrict__ pair_to_row) {
  __shared__ PermSmem sm;
  zero_hist(sm);
  __syncthreads();
  if (threadIdx.x < E) sm.cursor[threadIdx.x] = ws[(size_t)blockIdx.x * E + threadIdx.x];
  __syncthreads();
  scatter_round(sm, ids, P, E, blockIdx.x * kPermThreads, sorted_pair, pair_to_row);
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

size_t permute_workspace_bytes(int P, int E) {
  if (P <= kPermThreads) return 0;
  const size_t chunks = ((size_t)P + kPermThreads - 1) / kPermThreads;
  return (chunks * E * sizeof(int32_t) + 255) & ~(size_t)255;
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_to_row, void* ws, hipStream_t s) {
  if (P <= kPermThreads) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, P, E, offsets, sorted_pair,
                       pair_to_row);
    return hipGetLastError();
  }
  const int chunks = (P + kPermThreads - 1) / kPermThreads;
  int32_t* w = reinterpret_cast<int32_t*>(ws);
  hipLaunchKernelGGL(permute_count_kernel, dim3(chunks), dim3(kPermThreads), 0, s, ids, P, E, w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kPermThreads), 0, s, chunks, E, w, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(chunks), dim3(kPermThreads), 0, s, ids, P, E, w, sorted_pair,
                     pair_to_row);
  return hipGetLastError();
}

}  // namespace moe
