// Router gate projection upstream of the top-k router (gfx950):
//   logits[t][e] = sum_c x[t][c] * W_r[e][c] + bias[e]
// x and W_r are bf16, so every product is exact in fp32; sums are fp32 in a
// fixed order.  The router has to run before any expert can be read ("DeepSeek
// V4.1 Flash Q4 / 27 September 2026", "30 September follow-up: prefill"), so
// its cost sits in front of the expert streams of every layer.
//
// Two kernels, by batch size:
//  * a few tokens (decode, a verify batch): one workgroup per expert row.  Its
//    four wavefronts hold interleaved 512-element steps of the row in
//    registers (one 16-byte load per lane and step) and run the tokens past
//    them in groups; a wavefront's partial is reduced with DPP/permlane, the
//    four partials are added in wavefront order.  The top-k then runs as the
//    router kernel on the written logits (a token's k experts need all E
//    logits, which here come from E different workgroups).
//  * a chunk of tokens (prefill): a skinny GEMM on V_MFMA_F32_16X16X32_BF16.
//    A workgroup takes 32 tokens (two 16-row A fragments) against every
//    expert; each of its eight wavefronts owns every eighth 16-row fragment
//    of W_r.  K runs in chunks of 64 with a ring of register sets in flight.
//    With E <= 448 the 32 x E logits are also staged in LDS and the same
//    workgroup routes its tokens (the router of route_core.cuh), so the
//    projection and the top-k are one kernel.
// In both, lane (r, g) of a fragment supplies 16 consecutive bf16 of row r at
// element 64c + 16g of chunk c, two K-steps of eight each; A and B use the
// same K order, so the MFMA sums the plain dot product.
#include "common.cuh"
#include "kernels.h"
#include "route_core.cuh"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// ---------------------------------------------------------------------------
// GEMV: one workgroup per expert row
// ---------------------------------------------------------------------------

constexpr int kGvThreads = 256;

// 8 bf16 of W_r times 8 bf16 of x added to acc (products exact, fp32 sums in order).
__device__ __forceinline__ float dot8_bf16(const uint4& w, const uint4& x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc,
                                        false);
  return acc;
}

// S: 512-element steps per wavefront (wavefront w takes steps w, w+4, ...),
// TG: tokens per register group.
template <int S, int TG>
__global__ __launch_bounds__(kGvThreads) void router_gemv_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                                 const uint16_t* __restrict__ wr, int E,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ logits) {
  __shared__ float part[4][TG];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* row = wr + (size_t)e * H;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  int col[S];
  uint4 wv[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    col[i] = (wave + 4 * i) * 512 + 8 * lane;
    wv[i] = col[i] < H ? *reinterpret_cast<const uint4*>(row + col[i]) : zero;
  }
  const float b = bias ? bias[e] : 0.f;
  for (int t0 = 0; t0 < T; t0 += TG) {
    uint4 xv[TG][S];
#pragma unroll
    for (int j = 0; j < TG; ++j)
#pragma unroll
      for (int i = 0; i < S; ++i)
        xv[j][i] = (t0 + j < T && col[i] < H)
                       ? *reinterpret_cast<const uint4*>(x + (size_t)(t0 + j) * H + col[i])
                       : zero;
    float acc[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      acc[j] = 0.f;
#pragma unroll
      for (int i = 0; i < S; ++i) acc[j] = dot8_bf16(wv[i], xv[j][i], acc[j]);
      acc[j] = wave_sum_dpp(acc[j]);
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < TG; ++j) part[wave][j] = acc[j];
    }
    __syncthreads();
    if (threadIdx.x < TG && t0 + (int)threadIdx.x < T) {
      const int j = threadIdx.x;
      const float s = (part[0][j] + part[1][j]) + (part[2][j] + part[3][j]);
      logits[(size_t)(t0 + j) * E + e] = s + b;
    }
    __syncthreads();  // part is rewritten by the next token group
  }
}

// ---------------------------------------------------------------------------
// MFMA: 32 tokens x every expert per workgroup, optional in-kernel top-k
// ---------------------------------------------------------------------------

constexpr int kRmThreads = 512;   // eight wavefronts, two per SIMD
constexpr int kRmWaves = kRmThreads / 64;
constexpr int kRmTok = 32;        // tokens per workgroup
constexpr int kRmFusedMaxE = 448; // 32 x (E + 1) fp32 logits fit the LDS stage
constexpr int kRmStride = kRmFusedMaxE + 1;

template <int NF>
struct RmChunk {
  uint4_t a[2][2];   // [token fragment][K-step]
  uint4_t b[NF][2];  // [expert fragment][K-step]
};

template <int NF, int RING, bool FUSED>
__global__ __launch_bounds__(kRmThreads, 1) void router_mfma_kernel(
    const uint16_t* __restrict__ x, int T, int H, const uint16_t* __restrict__ wr, int E,
    const float* __restrict__ bias, float* __restrict__ logits, int k, const int32_t* __restrict__ e2s,
    int32_t* __restrict__ ids, float* __restrict__ tw) {
  __shared__ float lt[FUSED ? kRmTok * kRmStride : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kRmTok;
  const uint32_t rowb = (uint32_t)H * 2u;
  const rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)T * rowb));
  const rsrc_t wrr = make_rsrc(wr, (uint32_t)((size_t)E * rowb));
  uint32_t va[2], vb[NF];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int tok = t0 + 16 * m + q16;
    va[m] = tok < T ? (uint32_t)tok * rowb + 32u * g : kOob;  // rows past the batch read zeros
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int er = 16 * (wave + kRmWaves * j) + q16;
    vb[j] = er < E ? (uint32_t)er * rowb + 32u * g : kOob;    // rows past the experts read zeros
  }
  const int nch = H / 64;  // a multiple of RING (H % 256 == 0, RING <= 4)
  auto load = [&](RmChunk<NF>& r, int c) {
    const uint32_t o = 128u * (uint32_t)c;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < 2; ++t) r.a[m][t] = bload16(xr, va[m] + o + 16u * t);
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int t = 0; t < 2; ++t) r.b[j][t] = bload16(wrr, vb[j] + o + 16u * t);
  };
  f4v acc[2][NF];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[m][j] = f4v{0.f, 0.f, 0.f, 0.f};
  RmChunk<NF> ring[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r) load(ring[r], r);
  for (int c0 = 0; c0 < nch; c0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < NF; ++j)
            acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[r].a[m][t]),
                                                                as_bf16x8(ring[r].b[j][t]), acc[m][j], 0, 0, 0);
      // refill the set with the chunk RING ahead; past the end, the last chunk
      // again (in range, never multiplied), so no load sits behind a branch
      const int cn = c0 + r + RING;
      load(ring[r], cn < nch ? cn : nch - 1);
    }
  }
  // accumulator v of fragment pair (m, j): token t0 + 16m + 4g + v, expert 16(wave + 8j) + q16
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int er = 16 * (wave + kRmWaves * j) + q16;
    if (er >= E) continue;
    const float b = bias ? bias[er] : 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * m + 4 * g + v;
        const float l = acc[m][j][v] + b;
        if (t0 + r < T) logits[(size_t)(t0 + r) * E + er] = l;
        if (FUSED) lt[r * kRmStride + er] = l;
      }
  }
  if (FUSED) {
    __syncthreads();
    // wavefront w routes rows 4w .. 4w+3 of the tile from LDS
#pragma unroll
    for (int i = 0; i < kRmTok / kRmWaves; ++i) {
      const int r = (kRmTok / kRmWaves) * wave + i, t = t0 + r;
      if (t >= T) break;  // whole wavefront leaves together
      const RoutePick pick = route_token<8>(lt + r * kRmStride, E, k, e2s, lane);
      if (lane < k) {
        ids[(size_t)t * k + lane] = pick.expert;
        tw[(size_t)t * k + lane] = pick.weight;
      }
    }
  }
}

constexpr int kGemvMaxT = 64;  // larger batches take the MFMA kernel

hipError_t launch_gemv(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias, float* logits,
                       hipStream_t s) {
  const int S = (H + 2047) / 2048;
  const dim3 grid(E), block(kGvThreads);
#define MOE_GV(SS, TG) \
  hipLaunchKernelGGL((router_gemv_kernel<SS, TG>), grid, block, 0, s, x, T, H, wr, E, bias, logits)
  switch (S) {
    case 1: MOE_GV(1, 8); break;
    case 2: MOE_GV(2, 8); break;
    case 3: MOE_GV(3, 8); break;
    case 4: MOE_GV(4, 4); break;
    case 5: MOE_GV(5, 4); break;
    case 6: MOE_GV(6, 4); break;
    case 7: MOE_GV(7, 2); break;
    default: MOE_GV(8, 2); break;
  }
#undef MOE_GV
  return hipGetLastError();
}

// fused: also route (k, e2s, ids, tw) inside the kernel; needs E <= kRmFusedMaxE
hipError_t launch_mfma(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias, float* logits,
                       bool fused, int k, const int32_t* e2s, int32_t* ids, float* tw, hipStream_t s) {
  const int nfrag = (E + 15) / 16, need = (nfrag + kRmWaves - 1) / kRmWaves;
  const dim3 grid((T + kRmTok - 1) / kRmTok), block(kRmThreads);
#define MOE_RM(NF, RING, FU)                                                                                  \
  hipLaunchKernelGGL((router_mfma_kernel<NF, RING, FU>), grid, block, 0, s, x, T, H, wr, E, bias, logits, k, \
                     e2s, ids, tw)
  if (fused) {
    switch (need) {
      case 1: MOE_RM(1, 4, true); break;
      case 2: MOE_RM(2, 4, true); break;
      case 3: MOE_RM(3, 4, true); break;
      default: MOE_RM(4, 4, true); break;
    }
  } else {
    switch (need) {
      case 1: MOE_RM(1, 4, false); break;
      case 2: MOE_RM(2, 4, false); break;
      case 3: MOE_RM(3, 4, false); break;
      case 4: MOE_RM(4, 4, false); break;
      case 5:
      case 6: MOE_RM(6, 2, false); break;
      default: MOE_RM(8, 2, false); break;
    }
  }
#undef MOE_RM
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias,
                                float* logits, hipStream_t s) {
  if (T <= kGemvMaxT) return launch_gemv(x, T, H, wr, E, bias, logits, s);
  return launch_mfma(x, T, H, wr, E, bias, logits, false, 0, nullptr, nullptr, nullptr, s);
}

hipError_t launch_route_x(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias, int k,
                          const int32_t* e2s, float* logits, int32_t* ids, float* tw, hipStream_t s) {
  if (T > kGemvMaxT && E <= kRmFusedMaxE)
    return launch_mfma(x, T, H, wr, E, bias, logits, true, k, e2s, ids, tw, s);
  const hipError_t err = launch_router_logits(x, T, H, wr, E, bias, logits, s);
  if (err != hipSuccess) return err;
  return launch_route(logits, T, E, k, e2s, ids, tw, s);
}

}  // namespace moe
