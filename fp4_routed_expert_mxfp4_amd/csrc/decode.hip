// Decode expert FFN over MXFP4 experts (gfx950): memory-bound GEMV pair.
//
// The weight rows of the routed experts -- e2m1 codes with one UE8M0 scale
// per 32 weights, the checkpoint's own layout ("DeepSeek-V4.1-Flash on a
// single NVIDIA DGX Spark", intro and "Why it is built this way") -- are
// streamed once from HBM with 16-byte coalesced loads and decoded in
// registers.  Decode is judged against unquantised activations ("Fast
// single-box DeepSeek v4.1 Flash runtime", "Conventions": prefill and decode
// are separate arithmetic paths), so x stays bf16 and h stays fp32.
//
// Kernel 1 (gate/up + SwiGLU): one wavefront per weight row n of the bucket's
//   expert; lane l owns K-blocks l, l+64, ... (32 weights = 16 code bytes =
//   one scale each).  A block is decoded with v_cvt_scalef32_pk_bf16_fp4
//   (exact: e2m1 has two significant bits) and reduced against x with
//   v_dot2_f32_bf16 (bf16 x bf16 products are exact in fp32); the block sum
//   is multiplied by its scale 2^(e-127) in fp32.  g and u of row n are then
//   wave-reduced and h = silu(g) * u is written in fp32.
// Kernel 2 (down): the same row walk over W_down with h in fp32; the e2m1
//   codes are decoded to fp32 with v_cvt_scalef32_pk_f32_fp4 and the block
//   sums use fp32 FMAs.  y_pair row p = t*k + j is written once.
//
// Work items are (bucket, row tile); the workgroups walk them grid-stride so
// a launch sized for the largest bucket count also serves fewer buckets.  A
// bucket's tokens reuse the weight registers; a one-token bucket keeps its
// activations in registers for the whole row walk.
#include "common.cuh"
#include "kernels.h"
#include "route_core.cuh"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Compact list of the non-empty buckets, built by wavefront 0 into LDS.
struct Buckets {
  int n;
  int expert[kMaxExperts];
  int row0[kMaxExperts];
  int cnt[kMaxExperts];
};

__device__ void build_buckets(const int32_t* __restrict__ offsets, int E, Buckets& b) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    constexpr int CH = kMaxExperts / 64;
    int off[CH + 1];
#pragma unroll
    for (int i = 0; i <= CH; ++i) {
      const int e = lane * CH + i;
      off[i] = offsets[e < E ? e : E];
    }
    int n = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) n += (lane * CH + i < E && off[i + 1] > off[i]) ? 1 : 0;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    int pos = incl - n;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = lane * CH + i;
      if (e < E && off[i + 1] > off[i]) {
        b.expert[pos] = e;
        b.row0[pos] = off[i];
        b.cnt[pos] = off[i + 1] - off[i];
        ++pos;
      }
    }
    if (lane == 63) b.n = incl;
  }
  __syncthreads();
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t comp(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// Sum over one 32-weight block of e2m1(code) * x, x given as 32 bf16 in 4 x uint4.
__device__ __forceinline__ float block_dot_bf16(const uint4& c, const uint4 (&x)[4]) {
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t word = comp(c, q);
    const uint4 xv = x[q];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 0),
                                          __builtin_bit_cast(bf16x2_t, xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 1),
                                          __builtin_bit_cast(bf16x2_t, xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 2),
                                          __builtin_bit_cast(bf16x2_t, xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 3),
                                          __builtin_bit_cast(bf16x2_t, xv.w), acc, false);
  }
  return acc;
}

// Sum over one 32-weight block of e2m1(code) * h, h given as 32 fp32.
__device__ __forceinline__ float block_dot_f32(const uint4& c, const float4_t (&h)[8]) {
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t word = comp(c, q);
    const float4_t ha = h[2 * q], hb = h[2 * q + 1];
    float2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
    float2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
    float2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
    float2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
    acc = fmaf(w0.x, ha.x, acc);
    acc = fmaf(w0.y, ha.y, acc);
    acc = fmaf(w1.x, ha.z, acc);
    acc = fmaf(w1.y, ha.w, acc);
    acc = fmaf(w2.x, hb.x, acc);
    acc = fmaf(w2.y, hb.y, acc);
    acc = fmaf(w3.x, hb.z, acc);
    acc = fmaf(w3.y, hb.w, acc);
  }
  return acc;
}

__device__ __forceinline__ void load_x_blocks(const uint16_t* xt, int NB, int lane, int jb,
                                              uint4 (&xr)[4]) {
  const int kb = lane + 64 * jb;
  if (kb < NB) {
    const uint4* p = reinterpret_cast<const uint4*>(xt + kb * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) xr[q] = p[q];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) xr[q] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void load_h_blocks(const float* hr, int NB, int lane, int jb, float4_t (&hv)[8]) {
  const int kb = lane + 64 * jb;
  if (kb < NB) {
    const float4_t* p = reinterpret_cast<const float4_t*>(hr + kb * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) hv[q] = p[q];
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) hv[q] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
}

template <int JB>
__global__ __launch_bounds__(kThreads) void gateup_kernel(const uint16_t* __restrict__ x, int k, int E,
                                                          ExpertStore w, const int32_t* __restrict__ e2s,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_pair,
                                                          float* __restrict__ h, int rows_per_wave,
                                                          int tiles) {
  __shared__ Buckets bk;
  build_buckets(offsets, E, bk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = w.H, I = w.I, NB = H / 32;
  const size_t rowbytes = (size_t)H / 2;
  const int nitems = bk.n * tiles;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int b = item / tiles, tile = item - b * tiles;
    const int expert = bk.expert[b], row0 = bk.row0[b], cnt = bk.cnt[b];
    const int slot = e2s ? e2s[expert] : expert;
    if (slot < 0 || slot >= w.num_slots) continue;  // the down kernel writes zero rows
    const uint8_t* gc = w.wg + (size_t)slot * I * rowbytes;
    const uint8_t* uc = w.wu + (size_t)slot * I * rowbytes;
    const uint8_t* gs = w.sg + (size_t)slot * I * NB;
    const uint8_t* us = w.su + (size_t)slot * I * NB;
    const int n0 = (tile * kWaves + wave) * rows_per_wave;
    const int n1 = min(n0 + rows_per_wave, I);
    uint4 xr[JB][4];
    const bool single = (cnt == 1);
    if (single) {
      const int t = sorted_pair[row0] / k;
#pragma unroll
      for (int j = 0; j < JB; ++j) load_x_blocks(x + (size_t)t * H, NB, lane, j, xr[j]);
    }
    for (int n = n0; n < n1; ++n) {
      uint4 cg[JB], cu[JB];
      float sg[JB], su[JB];
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int kb = lane + 64 * j;
        if (kb < NB) {
          cg[j] = ld16(gc + n * rowbytes + kb * 16);
          cu[j] = ld16(uc + n * rowbytes + kb * 16);
          sg[j] = ue8m0_to_f32(gs[(size_t)n * NB + kb]);
          su[j] = ue8m0_to_f32(us[(size_t)n * NB + kb]);
        } else {
          cg[j] = cu[j] = make_uint4(0, 0, 0, 0);
          sg[j] = su[j] = 0.f;
        }
      }
      for (int r = 0; r < cnt; ++r) {
        if (!single) {
          const int t = sorted_pair[row0 + r] / k;
#pragma unroll
          for (int j = 0; j < JB; ++j) load_x_blocks(x + (size_t)t * H, NB, lane, j, xr[j]);
        }
        float ag = 0.f, au = 0.f;
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          ag = fmaf(block_dot_bf16(cg[j], xr[j]), sg[j], ag);
          au = fmaf(block_dot_bf16(cu[j], xr[j]), su[j], au);
        }
        ag = wave_sum(ag);
        au = wave_sum(au);
        if (lane == 0) h[(size_t)(row0 + r) * I + n] = swiglu_f32(ag, au);
      }
    }
  }
}

template <int JB>
__global__ __launch_bounds__(kThreads) void down_kernel(int k, int E, ExpertStore w,
                                                        const int32_t* __restrict__ e2s,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ sorted_pair,
                                                        const float* __restrict__ h, float* __restrict__ y,
                                                        int rows_per_wave, int tiles) {
  __shared__ Buckets bk;
  build_buckets(offsets, E, bk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = w.H, I = w.I, NB = I / 32;
  const size_t rowbytes = (size_t)I / 2;
  const int nitems = bk.n * tiles;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int b = item / tiles, tile = item - b * tiles;
    const int expert = bk.expert[b], row0 = bk.row0[b], cnt = bk.cnt[b];
    const int slot = e2s ? e2s[expert] : expert;
    const int m0 = (tile * kWaves + wave) * rows_per_wave;
    const int m1 = min(m0 + rows_per_wave, H);
    if (slot < 0 || slot >= w.num_slots) {
      for (int r = 0; r < cnt; ++r) {
        const int p = sorted_pair[row0 + r];
        for (int m = m0 + lane; m < m1; m += 64) y[(size_t)p * H + m] = 0.f;
      }
      continue;
    }
    const uint8_t* dc = w.wd + (size_t)slot * H * rowbytes;
    const uint8_t* ds = w.sd + (size_t)slot * H * NB;
    float4_t hv[JB][8];
    const bool single = (cnt == 1);
    if (single) {
#pragma unroll
      for (int j = 0; j < JB; ++j) load_h_blocks(h + (size_t)row0 * I, NB, lane, j, hv[j]);
    }
    for (int m = m0; m < m1; ++m) {
      uint4 c[JB];
      float s[JB];
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int kb = lane + 64 * j;
        if (kb < NB) {
          c[j] = ld16(dc + m * rowbytes + kb * 16);
          s[j] = ue8m0_to_f32(ds[(size_t)m * NB + kb]);
        } else {
          c[j] = make_uint4(0, 0, 0, 0);
          s[j] = 0.f;
        }
      }
      for (int r = 0; r < cnt; ++r) {
        if (!single) {
#pragma unroll
          for (int j = 0; j < JB; ++j) load_h_blocks(h + (size_t)(row0 + r) * I, NB, lane, j, hv[j]);
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < JB; ++j) acc = fmaf(block_dot_f32(c[j], hv[j]), s[j], acc);
        acc = wave_sum(acc);
        if (lane == 0) y[(size_t)sorted_pair[row0 + r] * H + m] = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fast paths for the model's shapes.
//
// Gate/up at H = 1024*J: the gate row n and the up row n together hold 2*H/32
// = 64*J blocks, so a row pair is exactly J full-wave 16-byte loads (lane l
// takes blocks l + 64*j of the concatenated pair) and no lane idles.  The
// blocks a lane touches are the same for every row, so its slice of x stays
// in registers.  R row pairs form a batch; the next batch's loads are issued
// before the current one is reduced (two register buffers), and the 2R
// partial sums of a batch are reduced with permlane swaps and DPP only.
//
// Down at I = 2048*M + 256*TAIL: a row has 64*M main blocks plus 8 tail
// blocks.  A batch is 8 rows: M full-wave loads per row for the main blocks,
// and one full-wave load for the 8 tails (lane l takes tail block l%8 of row
// l/8).  h stays in registers for a one-token bucket.
// ---------------------------------------------------------------------------

template <int J, int R>
struct GateUpBatch {
  uint4 c[R][J];
  uint32_t s[R][J];  // raw UE8M0 bytes, decoded when the batch is reduced
};

// Issue the loads of R row pairs starting at n0 (the caller guarantees n0 + R <= I).
template <int J, int R>
__device__ __forceinline__ void gu_load(GateUpBatch<J, R>& B, const uint8_t* const (&cp)[J],
                                        const uint8_t* const (&sp)[J], int n0, size_t rowbytes, int NB) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const size_t n = (size_t)(n0 + i);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      B.c[i][j] = ld16(cp[j] + n * rowbytes);
      B.s[i][j] = sp[j][n * NB];
    }
  }
}

// Reduce the batch for one token and store h for its R rows.
template <int J, int R>
__device__ __forceinline__ void gu_finish(const GateUpBatch<J, R>& B, const uint4 (&xr)[J][4], int lane,
                                          float* hrow, int n0) {
  constexpr int NB = 32 * J;
  float g[R], u[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    g[i] = 0.f;
    u[i] = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float d = block_dot_bf16(B.c[i][j], xr[j]) * ue8m0_to_f32(B.s[i][j]);
      if (64 * (j + 1) <= NB) {
        g[i] += d;                                  // all lanes in the gate row
      } else if (64 * j >= NB) {
        u[i] += d;                                  // all lanes in the up row
      } else {
        const bool gate = lane + 64 * j < NB;       // the load straddles the two rows
        g[i] += gate ? d : 0.f;
        u[i] += gate ? 0.f : d;
      }
    }
  }
  float gv[R], uv[R];
  if constexpr (R == 1) {
    float a = sum16(tswap32(g[0], u[0]));           // lanes 0-31: g, 32-63: u (16-lane partials)
    a = tswap16(a, a);
    gv[0] = lane_value(a, 0);
    uv[0] = lane_value(a, 32);
  } else {
    static_assert(R == 2, "gate/up batches of 1 or 2 row pairs");
    const float a0 = tswap32(g[0], g[1]);
    const float a1 = tswap32(u[0], u[1]);
    const float b = sum16(tswap16(a0, a1));         // rows: g0, u0, g1, u1
    gv[0] = lane_value(b, 0);
    uv[0] = lane_value(b, 16);
    gv[1] = lane_value(b, 32);
    uv[1] = lane_value(b, 48);
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (lane == i) hrow[n0 + i] = swiglu_f32(gv[i], uv[i]);
}

template <int J, int R>
__global__ __launch_bounds__(kThreads, 2) void gateup_fast_kernel(
    const uint16_t* __restrict__ x, int k, int E, ExpertStore w, const int32_t* __restrict__ e2s,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, float* __restrict__ h) {
  constexpr int NB = 32 * J;
  __shared__ Buckets bk;
  build_buckets(offsets, E, bk);
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int total_waves = gridDim.x * kWaves;
  const int I = w.I;
  const size_t rowbytes = (size_t)16 * NB;
  const int nbat = I / R;                 // I % R == 0 is checked at launch
  const int nbk = bk.n;
  int C = nbk > 0 ? total_waves / nbk : 1;
  if (C < 1) C = 1;
  const int cs = (nbat + C - 1) / C;
  const int units = nbk * C;
  for (int unit = gw; unit < units; unit += total_waves) {
    const int b = unit / C, c = unit - b * C;
    const int bat0 = c * cs, bat1 = min(bat0 + cs, nbat);
    if (bat0 >= bat1) continue;
    const int expert = bk.expert[b], row0 = bk.row0[b];
    const int slot = e2s ? e2s[expert] : expert;
    if (slot < 0 || slot >= w.num_slots) continue;  // the down kernel writes zero rows
    const uint8_t* cb[2] = {w.wg + (size_t)slot * I * rowbytes, w.wu + (size_t)slot * I * rowbytes};
    const uint8_t* sb[2] = {w.sg + (size_t)slot * I * NB, w.su + (size_t)slot * I * NB};
    const uint8_t* cp[J];
    const uint8_t* sp[J];
    int xblk[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int f = lane + 64 * j, mat = f >= NB ? 1 : 0, blk = f - mat * NB;
      cp[j] = cb[mat] + blk * 16;
      sp[j] = sb[mat] + blk;
      xblk[j] = blk;
    }
    uint4 xr[J][4];
    auto load_x = [&](int t) {
      const uint16_t* xt = x + (size_t)t * NB * 32;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint4* p = reinterpret_cast<const uint4*>(xt + xblk[j] * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) xr[j][q] = p[q];
      }
    };
    // one token per bucket: x stays in registers, two batches in flight
    load_x(sorted_pair[row0] / k);
    float* hrow = h + (size_t)row0 * I;
    GateUpBatch<J, R> A, Bn;
    gu_load(A, cp, sp, bat0 * R, rowbytes, NB);
    for (int bat = bat0; bat < bat1; bat += 2) {
      const bool has1 = bat + 1 < bat1;
      if (has1) gu_load(Bn, cp, sp, (bat + 1) * R, rowbytes, NB);
      gu_finish(A, xr, lane, hrow, bat * R);
      if (bat + 2 < bat1) gu_load(A, cp, sp, (bat + 2) * R, rowbytes, NB);
      if (has1) gu_finish(Bn, xr, lane, hrow, (bat + 1) * R);
    }

  }
}

template <int M, bool TAIL>
struct DownBatch {
  uint4 c[8][M > 0 ? M : 1];
  uint32_t s[8][M > 0 ? M : 1];  // raw UE8M0 bytes
  uint4 ct;
  uint32_t st;
};

template <int M, bool TAIL>
__device__ __forceinline__ void dn_load(DownBatch<M, TAIL>& B, const uint8_t* dc, const uint8_t* ds, int m0,
                                        int lane, size_t rowbytes, int NB) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
      const size_t row = (size_t)(m0 + i);
      B.c[i][mm] = ld16(dc + row * rowbytes + (size_t)(64 * mm + lane) * 16);
      B.s[i][mm] = ds[row * NB + 64 * mm + lane];
    }
  }
  if (TAIL) {
    const size_t row = (size_t)(m0 + (lane >> 3));
    const int blk = 64 * M + (lane & 7);
    B.ct = ld16(dc + row * rowbytes + (size_t)blk * 16);
    B.st = ds[row * NB + blk];
  }
}

template <int M, bool TAIL>
__device__ __forceinline__ void dn_finish(const DownBatch<M, TAIL>& B, const float4_t (&hm)[M > 0 ? M : 1][8],
                                          const float4_t (&ht)[8], int lane, float* yrow, int m0) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = 0.f;
#pragma unroll
    for (int mm = 0; mm < M; ++mm) v[i] = fmaf(block_dot_f32(B.c[i][mm], hm[mm]), ue8m0_to_f32(B.s[i][mm]), v[i]);
  }
  // 8 row partials -> lanes 8g..8g+7 hold partials of row g
  const float a0 = tswap32(v[0], v[4]), a1 = tswap32(v[1], v[5]);
  const float a2 = tswap32(v[2], v[6]), a3 = tswap32(v[3], v[7]);
  const float b0 = tswap16(a0, a2), b1 = tswap16(a1, a3);
  float c = tswap8(b0, b1, lane);
  if (TAIL) c += block_dot_f32(B.ct, ht) * ue8m0_to_f32(B.st);  // this lane's tail block is in row lane/8
  c = sum8(c);
  if ((lane & 7) == 0) yrow[m0 + (lane >> 3)] = c;
}

template <int M, bool TAIL>
__global__ __launch_bounds__(kThreads, 2) void down_fast_kernel(
    int k, int E, ExpertStore w, const int32_t* __restrict__ e2s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, const float* __restrict__ h, float* __restrict__ y) {
  constexpr int NB = 64 * M + (TAIL ? 8 : 0);
  constexpr int MM = M > 0 ? M : 1;
  __shared__ Buckets bk;
  build_buckets(offsets, E, bk);
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int total_waves = gridDim.x * kWaves;
  const int H = w.H, I = w.I;
  const size_t rowbytes = (size_t)16 * NB;
  const int nbat = H / 8;
  const int nbk = bk.n;
  int C = nbk > 0 ? total_waves / nbk : 1;
  if (C < 1) C = 1;
  const int cs = (nbat + C - 1) / C;
  const int units = nbk * C;
  for (int unit = gw; unit < units; unit += total_waves) {
    const int b = unit / C, c = unit - b * C;
    const int bat0 = c * cs, bat1 = min(bat0 + cs, nbat);
    if (bat0 >= bat1) continue;
    const int expert = bk.expert[b], row0 = bk.row0[b];
    const int slot = e2s ? e2s[expert] : expert;
    if (slot < 0 || slot >= w.num_slots) {
      float* yr = y + (size_t)sorted_pair[row0] * H;
      for (int m = bat0 * 8 + lane; m < bat1 * 8; m += 64) yr[m] = 0.f;
      continue;
    }
    const uint8_t* dc = w.wd + (size_t)slot * H * rowbytes;
    const uint8_t* ds = w.sd + (size_t)slot * H * NB;
    float4_t hm[MM][8], ht[8];
    auto load_h = [&](int row) {
      const float* hr = h + (size_t)row * I;
#pragma unroll
      for (int mm = 0; mm < M; ++mm) {
        const float4_t* p = reinterpret_cast<const float4_t*>(hr + (64 * mm + lane) * 32);
#pragma unroll
        for (int q = 0; q < 8; ++q) hm[mm][q] = p[q];
      }
      if (TAIL) {
        const float4_t* p = reinterpret_cast<const float4_t*>(hr + (64 * M + (lane & 7)) * 32);
#pragma unroll
        for (int q = 0; q < 8; ++q) ht[q] = p[q];
      }
    };
    // one token per bucket: h stays in registers, two batches in flight
    load_h(row0);
    float* yrow = y + (size_t)sorted_pair[row0] * H;
    DownBatch<M, TAIL> A, Bn;
    dn_load(A, dc, ds, bat0 * 8, lane, rowbytes, NB);
    for (int bat = bat0; bat < bat1; bat += 2) {
      const bool has1 = bat + 1 < bat1;
      if (has1) dn_load(Bn, dc, ds, (bat + 1) * 8, lane, rowbytes, NB);
      dn_finish(A, hm, ht, lane, yrow, bat * 8);
      if (bat + 2 < bat1) dn_load(A, dc, ds, (bat + 2) * 8, lane, rowbytes, NB);
      if (has1) dn_finish(Bn, hm, ht, lane, yrow, (bat + 1) * 8);
    }

  }
}

// ---------------------------------------------------------------------------
// Fused one-token decode layer: two launches instead of five.
//
// K1 (route + gate/up): every workgroup routes the token itself (one
//   wavefront, the router of route_core.cuh), so no workgroup waits for
//   another; the buckets of a one-token batch are its k experts in ascending
//   id.  Then the same gate/up row walk as gateup_fast_kernel writes h.
//   Workgroup 0 also publishes the routing for K2 and the caller.
// K2 (down + combine): one wavefront per routed expert over a slice of 24
//   output rows (three 8-row batches of down_fast_kernel's walk); the k rows
//   meet in LDS and are summed in ascending slot order exactly as
//   combine_kernel does, plus the residual, straight into the output.
// Per-row arithmetic is that of the separate kernels, so the result is
// bit-identical to route -> permute -> decode -> combine.
// ---------------------------------------------------------------------------

constexpr int kFusedMaxK = 8;
constexpr int kFusedRows = 24;

struct FusedRoute {
  int expert[kMaxTopK];       // bucket order: ascending expert id
  int slot[kMaxTopK];         // storage slot of each bucket's expert (-1: none)
  int row_of_pair[kMaxTopK];  // bucket row of slot j
  float w[kMaxTopK];          // weight of slot j
};

template <int NPL>
__device__ void fused_route(const float* __restrict__ logits, int E, int k, const int32_t* __restrict__ e2s,
                            int num_slots, FusedRoute& fr, FusedRoute* __restrict__ pub,
                            int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const RoutePick pick = route_token<NPL>(logits, E, k, e2s, lane);
    // rank of this slot's expert among the k picks (ties broken by slot)
    int r = 0;
    for (int i = 0; i < k; ++i) {
      const int ei = __shfl(pick.expert, i, 64);
      r += (ei < pick.expert || (ei == pick.expert && i < lane)) ? 1 : 0;
    }
    if (lane < k) {
      int sl = e2s ? e2s[pick.expert] : pick.expert;
      if (sl >= num_slots) sl = -1;
      fr.expert[r] = pick.expert;
      fr.slot[r] = sl;
      fr.row_of_pair[lane] = r;
      fr.w[lane] = pick.weight;
      if (blockIdx.x == 0) {
        topk_ids[lane] = pick.expert;
        topk_w[lane] = pick.weight;
        pub->expert[r] = pick.expert;
        pub->slot[r] = sl;
        pub->row_of_pair[lane] = r;
        pub->w[lane] = pick.weight;
      }
    }
  }
  __syncthreads();
}

template <int NPL, int J>
__global__ __launch_bounds__(kThreads, 2) void fused_gateup_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int E, int k, const int32_t* __restrict__ e2s,
    ExpertStore w, FusedRoute* __restrict__ pub, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    float* __restrict__ h) {
  constexpr int R = 2;
  constexpr int NB = 32 * J;
  __shared__ FusedRoute fr;
  fused_route<NPL>(logits, E, k, e2s, w.num_slots, fr, pub, topk_ids, topk_w);
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int total_waves = gridDim.x * kWaves;
  const int I = w.I;
  const size_t rowbytes = (size_t)16 * NB;
  const int nbat = I / R;
  int C = total_waves / k;
  if (C < 1) C = 1;
  const int cs = (nbat + C - 1) / C;
  const int units = k * C;
  // the token's x: lane l owns blocks (l + 64j) mod NB of the concatenated gate/up row
  uint4 xr[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int f = lane + 64 * j, blk = f >= NB ? f - NB : f;
    const uint4* px = reinterpret_cast<const uint4*>(x + blk * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) xr[j][q] = px[q];
  }
  for (int unit = gw; unit < units; unit += total_waves) {
    const int b = unit / C, c = unit - b * C;
    const int bat0 = c * cs, bat1 = min(bat0 + cs, nbat);
    if (bat0 >= bat1) continue;
    const int slot = fr.slot[b];
    if (slot < 0) continue;  // no stored expert: K2 contributes zero rows
    const uint8_t* cb[2] = {w.wg + (size_t)slot * I * rowbytes, w.wu + (size_t)slot * I * rowbytes};
    const uint8_t* sb[2] = {w.sg + (size_t)slot * I * NB, w.su + (size_t)slot * I * NB};
    const uint8_t* cp[J];
    const uint8_t* sp[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int f = lane + 64 * j, mat = f >= NB ? 1 : 0, blk = f - mat * NB;
      cp[j] = cb[mat] + blk * 16;
      sp[j] = sb[mat] + blk;
    }
    float* hrow = h + (size_t)b * I;
    GateUpBatch<J, R> A, Bn;
    gu_load(A, cp, sp, bat0 * R, rowbytes, NB);
    for (int bat = bat0; bat < bat1; bat += 2) {
      const bool has1 = bat + 1 < bat1;
      if (has1) gu_load(Bn, cp, sp, (bat + 1) * R, rowbytes, NB);
      gu_finish(A, xr, lane, hrow, bat * R);
      if (bat + 2 < bat1) gu_load(A, cp, sp, (bat + 2) * R, rowbytes, NB);
      if (has1) gu_finish(Bn, xr, lane, hrow, (bat + 1) * R);
    }
  }
}

template <int M, bool TAIL, bool kBf16Out>
__global__ __launch_bounds__(kFusedMaxK * 64) void fused_down_combine_kernel(
    int k, ExpertStore w, const FusedRoute* __restrict__ pub, const float* __restrict__ h,
    const uint16_t* __restrict__ residual, void* __restrict__ out) {
  constexpr int NB = 64 * M + (TAIL ? 8 : 0);
  constexpr int MM = M > 0 ? M : 1;
  __shared__ FusedRoute fr;
  __shared__ float ybuf[kFusedMaxK][kFusedRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kMaxTopK) {
    fr.expert[tid] = pub->expert[tid];
    fr.slot[tid] = pub->slot[tid];
    fr.row_of_pair[tid] = pub->row_of_pair[tid];
    fr.w[tid] = pub->w[tid];
  }
  __syncthreads();
  const int H = w.H, I = w.I;
  const int m0 = blockIdx.x * kFusedRows;
  const int nb = min(kFusedRows, H - m0) / 8;  // 8-row batches in this slice
  const int slot = fr.slot[wave];
  if (slot < 0) {
    if (lane < kFusedRows) ybuf[wave][lane] = 0.f;
  } else {
    const size_t rowbytes = (size_t)16 * NB;
    const uint8_t* dc = w.wd + (size_t)slot * H * rowbytes;
    const uint8_t* ds = w.sd + (size_t)slot * H * NB;
    float4_t hm[MM][8], ht[8];
    const float* hr = h + (size_t)wave * I;
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
      const float4_t* p = reinterpret_cast<const float4_t*>(hr + (64 * mm + lane) * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q) hm[mm][q] = p[q];
    }
    if (TAIL) {
      const float4_t* p = reinterpret_cast<const float4_t*>(hr + (64 * M + (lane & 7)) * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q) ht[q] = p[q];
    }
    DownBatch<M, TAIL> A, Bn;
    dn_load(A, dc, ds, m0, lane, rowbytes, NB);
    for (int bat = 0; bat < nb; bat += 2) {
      const bool has1 = bat + 1 < nb;
      if (has1) dn_load(Bn, dc, ds, m0 + (bat + 1) * 8, lane, rowbytes, NB);
      dn_finish(A, hm, ht, lane, ybuf[wave], bat * 8);
      if (bat + 2 < nb) dn_load(A, dc, ds, m0 + (bat + 2) * 8, lane, rowbytes, NB);
      if (has1) dn_finish(Bn, hm, ht, lane, ybuf[wave], (bat + 1) * 8);
    }
  }
  __syncthreads();
  if (tid < nb * 8) {
    const int m = m0 + tid;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(fr.w[j], ybuf[fr.row_of_pair[j]][tid], acc);
    if (residual) acc += bf16_bits_to_f32(residual[m]);
    if (kBf16Out)
      reinterpret_cast<uint16_t*>(out)[m] = f32_to_bf16_rne(acc);
    else
      reinterpret_cast<float*>(out)[m] = acc;
  }
}

template <int JB>
hipError_t launch_gateup_jb(dim3 grid, const uint16_t* x, int k, int E, const ExpertStore& w,
                            const int32_t* e2s, const int32_t* offsets, const int32_t* sorted_pair,
                            float* h, int rpw, int tiles, hipStream_t s) {
  hipLaunchKernelGGL(gateup_kernel<JB>, grid, dim3(kThreads), 0, s, x, k, E, w, e2s, offsets,
                     sorted_pair, h, rpw, tiles);
  return hipGetLastError();
}

template <int JB>
hipError_t launch_down_jb(dim3 grid, int k, int E, const ExpertStore& w, const int32_t* e2s,
                          const int32_t* offsets, const int32_t* sorted_pair, const float* h, float* y,
                          int rpw, int tiles, hipStream_t s) {
  hipLaunchKernelGGL(down_kernel<JB>, grid, dim3(kThreads), 0, s, k, E, w, e2s, offsets, sorted_pair, h,
                     y, rpw, tiles);
  return hipGetLastError();
}

int pick_rows_per_wave(int rows, int nb_max, int target_waves) {
  long total = (long)rows * nb_max;
  int rpw = (int)((total + target_waves - 1) / target_waves);
  return rpw < 1 ? 1 : (rpw > 64 ? 64 : rpw);
}

}  // namespace

bool fused_decode_supported(int T, int k, int E, int H, int I) {
  const int NB2 = I / 32, tail = NB2 % 64, M = NB2 / 64;
  return T == 1 && k <= kFusedMaxK && E <= kMaxExperts && H % 1024 == 0 && H / 1024 <= 6 &&
         (tail == 0 || tail == 8) && M <= 1 && (M > 0 || tail == 8);
}

size_t fused_decode_workspace_bytes(int k, int I) {
  return 512 + (((size_t)k * I * sizeof(float) + 255) & ~(size_t)255);
}

hipError_t launch_decode_fused(const float* logits, const uint16_t* x, int E, int k, const int32_t* e2s,
                               const ExpertStore& w, const uint16_t* residual, bool bf16_out, void* out,
                               int32_t* topk_ids, float* topk_w, void* ws, int phase, hipStream_t s) {
  FusedRoute* pub = reinterpret_cast<FusedRoute*>(ws);
  float* h = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + 512);
  const int J = w.H / 1024, npl = (E + 63) / 64;
  const dim3 g1(512), b1(kThreads);
  if (phase != 2) {
#define MOE_FGU(NP, JJ)                                                                                      \
  hipLaunchKernelGGL((fused_gateup_kernel<NP, JJ>), g1, b1, 0, s, logits, x, E, k, e2s, w, pub, topk_ids, topk_w, h)
#define MOE_FGU_J(NP)                                                                                        \
  switch (J) { case 1: MOE_FGU(NP, 1); break; case 2: MOE_FGU(NP, 2); break; case 3: MOE_FGU(NP, 3); break;  \
               case 4: MOE_FGU(NP, 4); break; case 5: MOE_FGU(NP, 5); break; default: MOE_FGU(NP, 6); break; }
  if (npl <= 1) { MOE_FGU_J(1) } else if (npl <= 2) { MOE_FGU_J(2) } else if (npl <= 4) { MOE_FGU_J(4) }
  else if (npl <= 8) { MOE_FGU_J(8) } else { MOE_FGU_J(16) }
#undef MOE_FGU_J
#undef MOE_FGU
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || phase == 1) return err;
  }
  const int NB2 = w.I / 32, M = NB2 / 64, tail = NB2 % 64;
  const dim3 g2((w.H + kFusedRows - 1) / kFusedRows), b2(k * 64);
#define MOE_FDC(MM, TT, BF)                                                                                  \
  hipLaunchKernelGGL((fused_down_combine_kernel<MM, TT, BF>), g2, b2, 0, s, k, w, pub, h, residual, out)
  if (tail == 8) {
    if (M == 0) { if (bf16_out) MOE_FDC(0, true, true); else MOE_FDC(0, true, false); }
    else { if (bf16_out) MOE_FDC(1, true, true); else MOE_FDC(1, true, false); }
  } else {
    if (bf16_out) MOE_FDC(1, false, true); else MOE_FDC(1, false, false);
  }
#undef MOE_FDC
  return hipGetLastError();
}

size_t decode_workspace_bytes(int T, int k, int I) {
  size_t b = (size_t)T * k * I * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

hipError_t launch_decode(const uint16_t* x, int T, int k, int E, const ExpertStore& w,
                         const int32_t* e2s, const int32_t* offsets, const int32_t* sorted_pair,
                         float* y_pair, void* ws, int phase, hipStream_t s) {
  const int P = T * k;
  const int nb_max = P < E ? P : E;
  float* h = reinterpret_cast<float*>(ws);
  const int target = 2048;  // wavefronts: ~8 per CU on 256 CUs
  const dim3 fast_grid(512);
  hipError_t err = hipSuccess;

  if (phase != 2) {
    const int J = w.H / 1024;
    if (T == 1 && w.H % 1024 == 0 && J >= 1 && J <= 6 && w.I % 2 == 0) {
#define MOE_GU(JJ)                                                                                 \
  case JJ:                                                                                         \
    hipLaunchKernelGGL((gateup_fast_kernel<JJ, 2>), fast_grid, dim3(kThreads), 0, s, x, k, E, w, e2s, \
                       offsets, sorted_pair, h);                                                   \
    break;
      switch (J) { MOE_GU(1) MOE_GU(2) MOE_GU(3) MOE_GU(4) MOE_GU(5) MOE_GU(6) }
#undef MOE_GU
      err = hipGetLastError();
    } else {
      const int jb1 = (w.H / 32 + 63) / 64;
      const int rpw = pick_rows_per_wave(w.I, nb_max, target);
      const int tiles = (w.I + kWaves * rpw - 1) / (kWaves * rpw);
      const long items = (long)tiles * nb_max;
      const dim3 grid((unsigned)(items < 4096 ? items : 4096));
      switch (jb1) {
        case 1: err = launch_gateup_jb<1>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        case 2: err = launch_gateup_jb<2>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        case 3: err = launch_gateup_jb<3>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        case 4: err = launch_gateup_jb<4>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        case 5: err = launch_gateup_jb<5>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        case 6: err = launch_gateup_jb<6>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        case 7: err = launch_gateup_jb<7>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        case 8: err = launch_gateup_jb<8>(grid, x, k, E, w, e2s, offsets, sorted_pair, h, rpw, tiles, s); break;
        default: return hipErrorInvalidValue;
      }
    }
  }
  if (err != hipSuccess || phase == 1) return err;

  const int NB2 = w.I / 32, M = NB2 / 64, tail = NB2 % 64;
  if (T == 1 && (tail == 0 || tail == 8) && M <= 1 && (M > 0 || tail == 8)) {
#define MOE_DN(MM, TT)                                                                                  \
  hipLaunchKernelGGL((down_fast_kernel<MM, TT>), fast_grid, dim3(kThreads), 0, s, k, E, w, e2s, offsets, \
                     sorted_pair, h, y_pair)
    if (tail == 8) {
      if (M == 0) { MOE_DN(0, true); } else { MOE_DN(1, true); }
    } else {
      MOE_DN(1, false);
    }
#undef MOE_DN
    return hipGetLastError();
  }
  const int jb2 = (NB2 + 63) / 64;
  const int rpw = pick_rows_per_wave(w.H, nb_max, target);
  const int tiles = (w.H + kWaves * rpw - 1) / (kWaves * rpw);
  const long items = (long)tiles * nb_max;
  const dim3 grid((unsigned)(items < 4096 ? items : 4096));
  switch (jb2) {
    case 1: return launch_down_jb<1>(grid, k, E, w, e2s, offsets, sorted_pair, h, y_pair, rpw, tiles, s);
    case 2: return launch_down_jb<2>(grid, k, E, w, e2s, offsets, sorted_pair, h, y_pair, rpw, tiles, s);
    case 3: return launch_down_jb<3>(grid, k, E, w, e2s, offsets, sorted_pair, h, y_pair, rpw, tiles, s);
    case 4: return launch_down_jb<4>(grid, k, E, w, e2s, offsets, sorted_pair, h, y_pair, rpw, tiles, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
