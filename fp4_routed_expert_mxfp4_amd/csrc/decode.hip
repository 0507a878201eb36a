// One-token decode FFN over MXFP4 experts (gfx950): memory-bound GEMV pair.
//
// The weight rows of the routed experts -- e2m1 codes with one UE8M0 scale
// per 32 weights, the checkpoint's own layout ("DeepSeek-V4.1-Flash on a
// single NVIDIA DGX Spark", intro and "Why it is built this way") -- are
// streamed once from HBM with 16-byte coalesced loads and decoded in
// registers.  Decode is judged against unquantised activations ("Fast
// single-box DeepSeek v4.1 Flash runtime", "Conventions": prefill and decode
// are separate arithmetic paths), so x stays bf16 and h stays fp32.
//
// A block of 32 codes is decoded with v_cvt_scalef32_pk_bf16_fp4 (exact:
// e2m1 has two significant bits) and reduced against x with v_dot2_f32_bf16
// (bf16 x bf16 products are exact in fp32); the block sum is multiplied by
// its scale 2^(e-127) in fp32.  The down projection decodes to fp32
// (v_cvt_scalef32_pk_f32_fp4) and sums with fp32 FMAs against h.
//
// These kernels serve one token at the model's shapes (a bucket holds that
// token once, or several times for a repeated expert id);
// launch_decode sends every other shape and every batch of two or more tokens
// to the bf16 MFMA kernels of decode_mt.hip.  The fused layer kernels below
// also route in-kernel and combine in the down kernel.
#include "common.cuh"
#include "kernels.h"
#include "route_core.cuh"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;


// Weight rows are streamed once per call: non-temporal loads (measured 26.6 -> 25.0 us for
// the one-token route + gate/up kernel, whose 100 MB stream would otherwise churn the caches).
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

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
// nrep > 1: the bucket holds the same token nrep times (a repeated expert id
// of a one-token call); its rows are identical and all of them are stored.
template <int J, int R>
__device__ __forceinline__ void gu_finish(const GateUpBatch<J, R>& B, const uint4 (&xr)[J][4], int lane,
                                          float* hrow, int n0, int nrep = 1, int I = 0) {
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
  static_assert(R == 2, "gate/up batches of 2 row pairs");
  float gv[R], uv[R];
  const float a0 = tswap32(g[0], g[1]);
  const float a1 = tswap32(u[0], u[1]);
  const float b = sum16(tswap16(a0, a1));           // rows: g0, u0, g1, u1
  gv[0] = lane_value(b, 0);
  uv[0] = lane_value(b, 16);
  gv[1] = lane_value(b, 32);
  uv[1] = lane_value(b, 48);
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (lane == i) {
      const float v = swiglu_f32(gv[i], uv[i]);
      hrow[n0 + i] = v;
      for (int r = 1; r < nrep; ++r) hrow[(size_t)r * I + n0 + i] = v;
    }
}

template <int J, int R>
__global__ __launch_bounds__(kThreads, 2) void gateup_fast_kernel(
    const uint16_t* __restrict__ x, int k, int E, ExpertStore w, const int32_t* __restrict__ e2s,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, const uint8_t* __restrict__ run,
    float* __restrict__ h) {
  constexpr int NB = 32 * J;
  __shared__ Buckets bk;
  build_buckets(offsets, E, bk, run);
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
    // one token: x stays in registers, two batches in flight.  Every row of
    // the bucket is that token (cnt > 1 only for a repeated expert id), so
    // the rows are computed once and stored cnt times.
    load_x(sorted_pair[row0] / k);
    float* hrow = h + (size_t)row0 * I;
    const int nrep = bk.cnt[b];
    GateUpBatch<J, R> A, Bn;
    gu_load(A, cp, sp, bat0 * R, rowbytes, NB);
    for (int bat = bat0; bat < bat1; bat += 2) {
      const bool has1 = bat + 1 < bat1;
      if (has1) gu_load(Bn, cp, sp, (bat + 1) * R, rowbytes, NB);
      gu_finish(A, xr, lane, hrow, bat * R, nrep, I);
      if (bat + 2 < bat1) gu_load(A, cp, sp, (bat + 2) * R, rowbytes, NB);
      if (has1) gu_finish(Bn, xr, lane, hrow, (bat + 1) * R, nrep, I);
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

// extra, nextra: the further output rows of a bucket that holds one token
// several times (a repeated expert id of a one-token call), which get the
// same values as yrow; y is their base and H their row length.
template <int M, bool TAIL>
__device__ __forceinline__ void dn_finish(const DownBatch<M, TAIL>& B, const float4_t (&hm)[M > 0 ? M : 1][8],
                                          const float4_t (&ht)[8], int lane, float* yrow, int m0,
                                          const int32_t* extra = nullptr, int nextra = 0, float* y = nullptr,
                                          int H = 0) {
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
  if ((lane & 7) == 0) {
    yrow[m0 + (lane >> 3)] = c;
    for (int r = 0; r < nextra; ++r) y[(size_t)extra[r] * H + m0 + (lane >> 3)] = c;
  }
}

template <int M, bool TAIL>
__global__ __launch_bounds__(kThreads, 2) void down_fast_kernel(
    int k, int E, ExpertStore w, const int32_t* __restrict__ e2s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, const uint8_t* __restrict__ run, const float* __restrict__ h,
    float* __restrict__ y) {
  constexpr int NB = 64 * M + (TAIL ? 8 : 0);
  constexpr int MM = M > 0 ? M : 1;
  __shared__ Buckets bk;
  build_buckets(offsets, E, bk, run);
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
    const int nrep = bk.cnt[b];  // > 1 only for a repeated expert id of the one token
    if (slot < 0 || slot >= w.num_slots) {
      for (int r = 0; r < nrep; ++r) {
        float* yr = y + (size_t)sorted_pair[row0 + r] * H;
        for (int m = bat0 * 8 + lane; m < bat1 * 8; m += 64) yr[m] = 0.f;
      }
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
    // one token: h stays in registers, two batches in flight; the rows of a
    // repeated expert id are equal and stored once per pair
    load_h(row0);
    float* yrow = y + (size_t)sorted_pair[row0] * H;
    const int32_t* extra = sorted_pair + row0 + 1;
    DownBatch<M, TAIL> A, Bn;
    dn_load(A, dc, ds, bat0 * 8, lane, rowbytes, NB);
    for (int bat = bat0; bat < bat1; bat += 2) {
      const bool has1 = bat + 1 < bat1;
      if (has1) dn_load(Bn, dc, ds, (bat + 1) * 8, lane, rowbytes, NB);
      dn_finish(A, hm, ht, lane, yrow, bat * 8, extra, nrep - 1, y, H);
      if (bat + 2 < bat1) dn_load(A, dc, ds, (bat + 2) * 8, lane, rowbytes, NB);
      if (has1) dn_finish(Bn, hm, ht, lane, yrow, (bat + 1) * 8, extra, nrep - 1, y, H);
    }

  }
}

// ---------------------------------------------------------------------------
// Fused one-token decode layer: two launches instead of five.
//
// K1 (route + gate/up): every workgroup routes the token itself (one
//   wavefront, the router of route_core.cuh), so no workgroup waits for
//   another; the buckets of a one-token batch are its k experts in ascending
//   id.  Then gate/up batches of gateup_fast_kernel's arithmetic, dealt out
//   interleaved over all (expert, batch) pairs, write h.
//   Workgroup 0 also publishes the routing for K2 and the caller.
// K2 (down + combine): one wavefront per routed expert over a slice of 20
//   output rows (8-row batches of down_fast_kernel's arithmetic); the k rows
//   meet in LDS and are summed in ascending slot order exactly as
//   combine_kernel does, plus the residual, straight into the output.
// Per-row arithmetic is that of the separate kernels, so the result is
// bit-identical to route -> permute -> decode -> combine.
// ---------------------------------------------------------------------------

constexpr int kFusedMaxK = 8;
constexpr int kFusedRows = 20;  // output rows per down workgroup: 256 workgroups at hidden 5120

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
      const int ei = __builtin_amdgcn_readlane(pick.expert, i);
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

// The gate/up work of the one-token layer: wavefront gw of total_waves takes
// a contiguous range of R-row-pair batches of one bucket's expert and writes
// h for those rows (bucket-major rows of h, I floats each).
template <int J>
__device__ __forceinline__ void fused_gateup_rows(const FusedRoute& fr, const uint16_t* __restrict__ x, int k,
                                                  const ExpertStore& w, float* __restrict__ h, int gw,
                                                  int total_waves, int lane) {
  constexpr int R = 2;
  constexpr int NB = 32 * J;
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
  // Batch slot q = batch q % nbat of bucket q / nbat.  Wavefront gw takes
  // slots gw, gw + total_waves, ...: consecutive batches of one wavefront lie
  // in different experts and rows, so each wavefront samples many regions of
  // HBM instead of streaming one contiguous range.
  int matj[J], blkj[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int f = lane + 64 * j;
    matj[j] = f >= NB ? 1 : 0;
    blkj[j] = f - matj[j] * NB;
  }
  struct Where {
    const uint8_t* cp[J];
    const uint8_t* sp[J];
    float* hrow;
    int n0;
    bool store;
  };
  auto where = [&](int q, Where& wh) {
    const int b = q / nbat, bat = q - b * nbat;
    const int slot = fr.slot[b];
    wh.store = slot >= 0;  // no stored expert: the down half contributes zero rows
    const size_t s0 = (size_t)(slot >= 0 ? slot : 0);
    const uint8_t* cb[2] = {w.wg + s0 * I * rowbytes, w.wu + s0 * I * rowbytes};
    const uint8_t* sb[2] = {w.sg + s0 * I * NB, w.su + s0 * I * NB};
#pragma unroll
    for (int j = 0; j < J; ++j) {
      wh.cp[j] = cb[matj[j]] + blkj[j] * 16;
      wh.sp[j] = sb[matj[j]] + blkj[j];
    }
    wh.hrow = h + (size_t)b * I;
    wh.n0 = bat * R;
  };
  (void)cs;
  (void)units;
  const int nslot = k * nbat;
  if (gw >= nslot) return;
  // One batch in flight per wavefront: the next batch's loads go out once this
  // one is reduced (with two in flight the step measured 0.25 us slower: fewer
  // loads queued per wavefront stream faster, and the CU's eight wavefronts
  // cover each other's waits).
  Where wa;
  GateUpBatch<J, R> A;
  for (int q = gw; q < nslot; q += total_waves) {
    where(q, wa);
    gu_load(A, wa.cp, wa.sp, wa.n0, rowbytes, NB);
    if (wa.store) gu_finish(A, xr, lane, wa.hrow, wa.n0);
  }
}

// The chain's weightless RMS norm of the token, folded into K1 (NORM): the
// sum of squares is taken exactly as rmsnorm_kernel takes it for one row --
// thread t of 256 accumulates elements 8t + 2048i in element order with fmaf,
// each wave's 64 partials are summed by the xor butterfly, and the four wave
// sums are added as (p0 + p1) + (p2 + p3) -- and every element is divided by
// the same r, so the normalised row is bit-identical to moe_rmsnorm_bf16's.
// Wavefront 0 routes meanwhile; wavefront 1 also takes wavefront 0's partials.
constexpr int kNormMaxH = 6144;  // the largest hidden of the one-token layer

__device__ __forceinline__ float norm_thread_sum(const uint16_t* __restrict__ x, int H, int t) {
  float ss = 0.f;
  for (int h = t * 8; h < H; h += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + h);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_bits_to_f32(q[i] & 0xFFFFu), b = bf16_bits_to_f32(q[i] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  return ss;
}

template <int NPL, int J, bool NORM>
__global__ __launch_bounds__(kThreads, 2) void fused_gateup_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int E, int k, const int32_t* __restrict__ e2s,
    ExpertStore w, FusedRoute* __restrict__ pub, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    float* __restrict__ h, float eps) {
  __shared__ FusedRoute fr;
  __shared__ __attribute__((aligned(16))) uint16_t xn[NORM ? kNormMaxH : 8];
  __shared__ float npart[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, H = w.H;
  if (NORM && wave > 0) {
    const float ss = wave_sum(norm_thread_sum(x, H, tid));
    if (lane == 0) npart[wave] = ss;
    if (wave == 1) {
      const float s0 = wave_sum(norm_thread_sum(x, H, lane));
      if (lane == 0) npart[0] = s0;
    }
  }
  fused_route<NPL>(logits, E, k, e2s, w.num_slots, fr, pub, topk_ids, topk_w);  // ends on a barrier
  const uint16_t* xs = x;
  if (NORM) {
    const float r = sqrtf(((npart[0] + npart[1]) + (npart[2] + npart[3])) / (float)H + eps);
    for (int e = tid * 8; e < H; e += 256 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + e);
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = bf16_bits_to_f32(q[i] & 0xFFFFu) / r, b = bf16_bits_to_f32(q[i] >> 16) / r;
        o[i] = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
      }
      *reinterpret_cast<uint4*>(xn + e) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    __syncthreads();
    xs = xn;
  }
  fused_gateup_rows<J>(fr, xs, k, w, h, blockIdx.x * kWaves + wave, gridDim.x * kWaves, lane);
}

__device__ __forceinline__ uint4 as_uint4(const uint4_t& v) { return make_uint4(v[0], v[1], v[2], v[3]); }

// One 8-row batch of the down stream with range-checked loads: rows at or
// past nvalid (and every row when on is false) read zeros at no memory cost.
template <int M, bool TAIL>
__device__ __forceinline__ void dn_load_rows(DownBatch<M, TAIL>& B, rsrc_t rc, rsrc_t rs, int m0, int nvalid,
                                             bool on, int lane, uint32_t rowbytes, int NB) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool v = on && i < nvalid;
    const uint32_t oc = v ? (uint32_t)(m0 + i) * rowbytes : kOob, os = v ? (uint32_t)((m0 + i) * NB) : kOob;
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
      B.c[i][mm] = as_uint4(bload16_nt(rc, oc + (uint32_t)(64 * mm + lane) * 16u));
      B.s[i][mm] = bload1(rs, os + (uint32_t)(64 * mm + lane));
    }
  }
  if (TAIL) {
    const int r = lane >> 3, blk = 64 * M + (lane & 7);
    const bool v = on && r < nvalid;
    B.ct = as_uint4(bload16_nt(rc, v ? (uint32_t)(m0 + r) * rowbytes + (uint32_t)blk * 16u : kOob));
    B.st = bload1(rs, v ? (uint32_t)((m0 + r) * NB + blk) : kOob);
  }
}

// K2: workgroup g takes output rows 20g .. 20g + 19, wavefront j the bucket j
// (one routed expert): two full 8-row batches and the first half of a third,
// all of whose loads are issued at once (no load waits for another), reduced
// with down_fast_kernel's per-row arithmetic.
template <int M, bool TAIL, bool kBf16Out>
__global__ __launch_bounds__(kFusedMaxK * 64) void fused_down_combine_kernel(
    int k, ExpertStore w, const FusedRoute* __restrict__ pub, const float* __restrict__ h,
    const uint16_t* __restrict__ residual, void* __restrict__ out) {
  constexpr int NB = 64 * M + (TAIL ? 8 : 0);
  constexpr int MM = M > 0 ? M : 1;
  constexpr int NBAT = (kFusedRows + 7) / 8;
  __shared__ FusedRoute fr;
  __shared__ float ybuf[kFusedMaxK][8 * NBAT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = w.H, I = w.I;
  if (tid < kMaxTopK) {
    fr.expert[tid] = pub->expert[tid];
    fr.slot[tid] = pub->slot[tid];
    fr.row_of_pair[tid] = pub->row_of_pair[tid];
    fr.w[tid] = pub->w[tid];
  }
  __syncthreads();
  const int m0 = blockIdx.x * kFusedRows;
  const int nrows = min(kFusedRows, H - m0);
  const int slot = fr.slot[wave];
  const bool on = slot >= 0;
  const uint32_t rowbytes = 16u * NB;
  const size_t s0 = (size_t)(on ? slot : 0);
  const rsrc_t rc = make_rsrc(w.wd + s0 * H * rowbytes, (uint32_t)H * rowbytes);
  const rsrc_t rs = make_rsrc(w.sd + s0 * H * NB, (uint32_t)(H * NB));
  // h of this wavefront's bucket and every weight row of the slice, all in flight together
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
  DownBatch<M, TAIL> B[NBAT];
#pragma unroll
  for (int t = 0; t < NBAT; ++t) dn_load_rows(B[t], rc, rs, m0 + 8 * t, nrows - 8 * t, on, lane, rowbytes, NB);
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first use
#pragma unroll
  for (int t = 0; t < NBAT; ++t) dn_finish(B[t], hm, ht, lane, ybuf[wave], 8 * t);
  // an expert without storage contributes zero rows (its h was never written)
  if (!on && lane < 8 * NBAT) ybuf[wave][lane] = 0.f;
  __syncthreads();
  if (tid < nrows) {
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
                               int32_t* topk_ids, float* topk_w, void* ws, int phase, hipStream_t s, bool norm,
                               float eps) {
  FusedRoute* pub = reinterpret_cast<FusedRoute*>(ws);
  float* h = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + 512);
  const int J = w.H / 1024, npl = (E + 63) / 64;
  const dim3 g1(512), b1(kThreads);
  if (phase != 2) {
#define MOE_FGU(NP, JJ)                                                                                      \
  if (norm)                                                                                                  \
    hipLaunchKernelGGL((fused_gateup_kernel<NP, JJ, true>), g1, b1, 0, s, logits, x, E, k, e2s, w, pub, topk_ids, \
                       topk_w, h, eps);                                                                      \
  else                                                                                                       \
    hipLaunchKernelGGL((fused_gateup_kernel<NP, JJ, false>), g1, b1, 0, s, logits, x, E, k, e2s, w, pub, topk_ids, \
                       topk_w, h, eps)
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
                         float* y_pair, void* ws, int phase, hipStream_t s, const uint8_t* run) {
  const int J = w.H / 1024, NB2 = w.I / 32, M = NB2 / 64, tail = NB2 % 64;
  const bool one_token_shape = T == 1 && w.H % 1024 == 0 && J >= 1 && J <= 6 && (tail == 0 || tail == 8) &&
                               M <= 1 && (M > 0 || tail == 8);
  if (!one_token_shape)  // both halves on the multi-token kernels (their h layout differs)
    return launch_decode_mt(x, T, k, E, w, e2s, offsets, sorted_pair, y_pair, ws, phase, s, run);
  float* h = reinterpret_cast<float*>(ws);
  const dim3 fast_grid(512);
  if (phase != 2) {
#define MOE_GU(JJ)                                                                                    \
  case JJ:                                                                                            \
    hipLaunchKernelGGL((gateup_fast_kernel<JJ, 2>), fast_grid, dim3(kThreads), 0, s, x, k, E, w, e2s, \
                       offsets, sorted_pair, run, h);                                                 \
    break;
    switch (J) { MOE_GU(1) MOE_GU(2) MOE_GU(3) MOE_GU(4) MOE_GU(5) MOE_GU(6) }
#undef MOE_GU
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || phase == 1) return err;
  }
#define MOE_DN(MM, TT)                                                                                  \
  hipLaunchKernelGGL((down_fast_kernel<MM, TT>), fast_grid, dim3(kThreads), 0, s, k, E, w, e2s, offsets, \
                     sorted_pair, run, h, y_pair)
  if (tail == 8) {
    if (M == 0) { MOE_DN(0, true); } else { MOE_DN(1, true); }
  } else {
    MOE_DN(1, false);
  }
#undef MOE_DN
  return hipGetLastError();
}

}  // namespace moe
