// Router gate projection upstream of the top-k router (gfx950):
//   logits[t][e] = sum_c x[t][c] * W_r[e][c] + bias[e]
// x and W_r are bf16, so every product is exact in fp32; sums are fp32 in a
// fixed order.  The router has to run before any expert can be read ("DeepSeek
// V4.1 Flash Q4 / 27 September 2026", "30 September follow-up: prefill"), so
// its cost sits in front of the expert streams of every layer.
//
// Two kernels, by batch size:
//  * a few tokens (decode, a verify batch): one workgroup per 16 expert rows
//    and every 16 tokens, on the same MFMA; its eight wavefronts take
//    interleaved K-steps, issue all their loads in one round trip, and add
//    their 16x16 partial tiles in LDS in wavefront order.
//  * a chunk of tokens (prefill): a GEMM on V_MFMA_F32_16X16X32_BF16 over
//    64-token x 128-expert tiles.  K runs in chunks of 64: both operands'
//    chunks are loaded once per workgroup with whole-line loads and shared
//    through LDS, with a ring of chunks in flight.  Splitting the experts
//    over workgroups keeps each CU's share of W_r reads to a third of W_r at
//    384 experts.
// The top-k then runs as the router kernel on the written logits (a token's
// k experts need all E logits, which come from several workgroups).
// A and B fragments always take the same K order, so the MFMA sums the plain
// dot product.
#include "common.cuh"
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// ---------------------------------------------------------------------------
// Few tokens: one workgroup per 16 expert rows, K split over eight wavefronts
// ---------------------------------------------------------------------------

constexpr int kSkThreads = 512;  // eight wavefronts: K-steps s = w (mod 8)
constexpr int kSkBlock = 20;     // K-steps (32 elements each) loaded per round trip

// A = 16 W_r rows (the expert fragment), B = 16 tokens; lane (r, g) supplies
// 8 bf16 of row / token r at element 32s + 8g of K-step s.  Every load of a
// block is issued before the block's MFMAs; steps past the wavefront's share
// and rows past E or T read zeros (buffer range), so nothing is branched.
// The eight partial 16x16 tiles meet in LDS and are added in wavefront order.
__global__ __launch_bounds__(kSkThreads) void router_skinny_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                                   const uint16_t* __restrict__ wr, int E,
                                                                   const float* __restrict__ bias,
                                                                   float* __restrict__ logits) {
  __shared__ float part[8][4 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q16 = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 16;
  const uint32_t rowb = (uint32_t)H * 2u;
  const rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)T * rowb));
  const rsrc_t wrr = make_rsrc(wr, (uint32_t)((size_t)E * rowb));
  const int ks = H / 256;  // K-steps per wavefront (H % 256 == 0)
  const uint32_t vw = e0 + q16 < E ? (uint32_t)(e0 + q16) * rowb + 16u * g : kOob;
  for (int t0 = 0; t0 < T; t0 += 16) {
    const uint32_t vx = t0 + q16 < T ? (uint32_t)(t0 + q16) * rowb + 16u * g : kOob;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int b0 = 0; b0 < ks; b0 += kSkBlock) {
      uint4_t wa[kSkBlock], xb[kSkBlock];
#pragma unroll
      for (int i = 0; i < kSkBlock; ++i) {
        const int st = wave + 8 * (b0 + i);  // this wavefront's K-step
        const uint32_t o = 64u * (uint32_t)st;
        const bool in = b0 + i < ks;
        wa[i] = bload16(wrr, in ? vw + o : kOob);
        xb[i] = bload16(xr, in ? vx + o : kOob);
      }
      __builtin_amdgcn_sched_barrier(0);  // the whole block's loads go out before its MFMAs
#pragma unroll
      for (int i = 0; i < kSkBlock; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[i]), as_bf16x8(xb[i]), acc, 0, 0, 0);
    }
    // accumulator v: expert e0 + 4g + v, token t0 + q16
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave][v * 64 + lane] = acc[v];
    __syncthreads();
    if (tid < 256) {
      const int v = tid >> 6, l = tid & 63;
      const int e = e0 + 4 * (l >> 4) + v, t = t0 + (l & 15);
      float sum = part[0][tid];
#pragma unroll
      for (int w = 1; w < 8; ++w) sum += part[w][tid];
      if (e < E && t < T) logits[(size_t)t * E + e] = sum + (bias ? bias[e] : 0.f);
    }
    __syncthreads();  // part is rewritten by the next token group
  }
}

// ---------------------------------------------------------------------------
// MFMA: a 64-token x 128-expert tile per workgroup
// ---------------------------------------------------------------------------

constexpr int kRmThreads = 512;  // eight wavefronts, two per SIMD
constexpr int kRmTok = 64;       // tokens per tile: four 16-row A fragments
constexpr int kRmExp = 128;      // experts per tile: eight 16-row W_r fragments
constexpr int kRmAStride = 144;  // bytes per staged token row: 128 + 16 (rows land on distinct banks)

// Lane (r, g) of a fragment supplies 16 consecutive bf16 of row r at element
// 64c + 16g of chunk c, two K-steps of eight each.
// Wavefront w = 4*tm + te takes token fragments 2tm, 2tm+1 and expert
// fragments te, te+4 of the tile.  Per chunk of 64 K, the tile's 64 token
// rows and 128 W_r rows (128 B each) are loaded once per workgroup -- every
// load instruction covers eight whole 128-byte lines -- and staged in LDS,
// from where each wavefront reads its fragments in MFMA order.  Ring slot s
// holds the thread's pieces of the next chunk = s (mod RING), staged one
// chunk before it is multiplied; every slot is refilled RING chunks ahead,
// so the in-order wait for one slot never drains the loads of the others.
template <int RING>
__global__ __launch_bounds__(kRmThreads, 1) void router_mfma_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                                    const uint16_t* __restrict__ wr, int E,
                                                                    const float* __restrict__ bias,
                                                                    float* __restrict__ logits) {
  __shared__ uint8_t sa[2][kRmTok * kRmAStride];  // the token rows' chunk, double-buffered
  __shared__ uint8_t sb[2][kRmExp * kRmAStride];  // the W_r rows' chunk, double-buffered
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q16 = lane & 15, g = lane >> 4;
  const int tm = wave >> 2, te = wave & 3;
  const int t0 = blockIdx.x * kRmTok, e0 = blockIdx.y * kRmExp;
  const uint32_t rowb = (uint32_t)H * 2u;
  const rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)T * rowb));
  const rsrc_t wrr = make_rsrc(wr, (uint32_t)((size_t)E * rowb));
  // staging: thread tid moves 16-byte piece tid%8 of token row tid/8, and of
  // W_r rows tid/8 and 64 + tid/8; rows past the batch or the experts read zeros
  const int ar = tid >> 3, ap = tid & 7;
  const uint32_t vax = (t0 + ar < T) ? (uint32_t)(t0 + ar) * rowb + 16u * ap : kOob;
  uint32_t vbx[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int er = e0 + 64 * h + ar;
    vbx[h] = er < E ? (uint32_t)er * rowb + 16u * ap : kOob;
  }
  const int nch = H / 64;  // a multiple of RING (H % 256 == 0, RING <= 4)
  uint4_t aring[RING], bring[RING][2];
  auto load = [&](int slot, int c) {
    const uint32_t o = 128u * (uint32_t)c;
    aring[slot] = bload16(xr, vax + o);
#pragma unroll
    for (int h = 0; h < 2; ++h) bring[slot][h] = bload16(wrr, vbx[h] + o);
  };
  auto stage = [&](int slot, int buf) {
    *reinterpret_cast<uint4_t*>(sa[buf] + ar * kRmAStride + 16 * ap) = aring[slot];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<uint4_t*>(sb[buf] + (64 * h + ar) * kRmAStride + 16 * ap) = bring[slot][h];
  };
  f4v acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RING; ++r) load(r, r);  // nch >= 4 >= RING
  stage(0, 0);
  load(0, min(RING, nch - 1));
  for (int c0 = 0; c0 < nch; c0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int c = c0 + r, s1 = (r + 1) % RING;
      // chunk c sits in buffers c&1 (c0 is even, so that is r&1); buffers (c+1)&1 are free
      __syncthreads();
      stage(s1, (r + 1) & 1);
      load(s1, min(c + 1 + RING, nch - 1));  // past the end: the last chunk again (in range, never used)
      __builtin_amdgcn_sched_barrier(0);     // these loads go out before the LDS reads and MFMAs
      uint4_t af[2][2], bf[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          af[m][t] = *reinterpret_cast<const uint4_t*>(sa[r & 1] + (16 * (2 * tm + m) + q16) * kRmAStride + 32 * g +
                                                       16 * t);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          bf[j][t] = *reinterpret_cast<const uint4_t*>(sb[r & 1] + (16 * (te + 4 * j) + q16) * kRmAStride + 32 * g +
                                                       16 * t);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[m][t]), as_bf16x8(bf[j][t]), acc[m][j],
                                                                0, 0, 0);
    }
  }
  // accumulator v of fragment pair (m, j): token t0 + 16(2tm + m) + 4g + v,
  // expert e0 + 16(te + 4j) + q16
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int er = e0 + 16 * (te + 4 * j) + q16;
    if (er >= E) continue;
    const float b = bias ? bias[er] : 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 16 * (2 * tm + m) + 4 * g + v;
        if (t < T) logits[(size_t)t * E + er] = acc[m][j][v] + b;
      }
  }
}

constexpr int kSkinnyMaxT = 64;  // larger batches take the tiled kernel

hipError_t launch_skinny(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias,
                         float* logits, hipStream_t s) {
  hipLaunchKernelGGL(router_skinny_kernel, dim3((E + 15) / 16), dim3(kSkThreads), 0, s, x, T, H, wr, E, bias, logits);
  return hipGetLastError();
}

hipError_t launch_mfma(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias, float* logits,
                       hipStream_t s) {
  const dim3 grid((T + kRmTok - 1) / kRmTok, (E + kRmExp - 1) / kRmExp), block(kRmThreads);
  hipLaunchKernelGGL((router_mfma_kernel<4>), grid, block, 0, s, x, T, H, wr, E, bias, logits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias,
                                float* logits, hipStream_t s) {
  if (T <= kSkinnyMaxT) return launch_skinny(x, T, H, wr, E, bias, logits, s);
  return launch_mfma(x, T, H, wr, E, bias, logits, s);
}

hipError_t launch_route_x(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias, int k,
                          const int32_t* e2s, float* logits, int32_t* ids, float* tw, hipStream_t s) {
  const hipError_t err = launch_router_logits(x, T, H, wr, E, bias, logits, s);
  if (err != hipSuccess) return err;
  return launch_route(logits, T, E, k, e2s, ids, tw, s);
}

}  // namespace moe
