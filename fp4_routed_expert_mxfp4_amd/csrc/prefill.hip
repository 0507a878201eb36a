// Prefill expert FFN on gfx950 block-scaled MFMA (MXFP6 activations x MXFP4 experts).
//
// Prefill is its own arithmetic path, judged against its own reference
// ("Fast single-box DeepSeek v4.1 Flash runtime", "Conventions"), with the
// activations quantised as the DGX Spark engine's act-quant switch does
// ("Reproduce the checks").  The activations are MXFP6 (e2m3 + one UE8M0
// scale per 32): with e2m1 weights every 32-term block sum of
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 is exact (e2m3 x e2m1 products need at
// most 10 bits, inside the instruction's block fixed point), and e2m3 runs at
// the FP4/FP6 rate.
//
//   P0  quant_x:  x bf16 [T][H] -> xq [T][H/32][24 B] + xs [T][H/32]
//   P1  gateup:   per bucket tile: g = W_gate.x, u = W_up.x (MFMA, fp32),
//                 h = silu(g)*u, h -> MXFP6 into hq/hs (sorted-row order)
//   P2  down:     per bucket tile: y = W_down.h (MFMA, fp32) -> y_pair row p
//
// GEMM tiles are 128 (bucket rows) x 128 (weight rows) with K chunks of 128
// (four 32-blocks) double-buffered through LDS; four wavefronts each own a
// 64 x 64 sub-tile as 2 x 2 MFMA 32x32x64 fragments.  Workgroups are
// persistent: the tile list (bucket, weight tile, row tile -- row tiles of
// one weight tile adjacent, so they share that weight tile in L2) is split
// into eight contiguous ranges, one per XCD.
#include "common.cuh"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPT = 256;           // threads per workgroup
constexpr int BM = 128;            // bucket rows per tile
constexpr int BK = 128;            // K per chunk (4 blocks)
constexpr int A_STRIDE = 104;      // LDS bytes per A row: 4 x 24 B blocks + 8 pad
constexpr int B_STRIDE = 80;       // LDS bytes per B row: 4 x 16 B blocks + 16 pad
constexpr int H_STRIDE = 65;       // fp32 words per row of the h staging buffer
constexpr int kGrid = 512;         // persistent workgroups (2 per CU)

typedef int i8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

// ---- MXFP6 (e2m3) quantiser, exact arithmetic -------------------------------

// 6-bit e2m3 code of t (already divided by the block scale), round to nearest
// even, saturating at 7.5.
__device__ __forceinline__ uint32_t e2m3_rne(float t) {
  const uint32_t sign = (__float_as_uint(t) >> 26) & 0x20u;
  const float a = fabsf(t);
  uint32_t code;
  if (a < 1.0f) {
    code = (uint32_t)__builtin_rintf(a * 8.0f);  // 0..8; 8 is 1.0 (exponent 1, mantissa 0)
  } else {
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;  // (exp+127)<<3 | 3-bit mantissa
    code = r - (126u << 3);                                        // exponent bias 1
    code = code > 31u ? 31u : code;
  }
  return sign | code;
}

// One 32-element block -> 24 packed bytes (code i at bits 6i..6i+5) + scale byte.
// Block exponent X = floor(log2 amax) - 2 (+1 when the significand of amax
// exceeds 1.875), clamped to [-127, 127]; amax == 0 gives scale 0, codes 0.
__device__ __forceinline__ void q6_block(const float (&v)[32], uint32_t (&pk)[6], uint32_t& sbyte) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int w = 0; w < 6; ++w) pk[w] = 0u;
  if (amax == 0.f) {
    sbyte = 0u;
    return;
  }
  const uint32_t ab = __float_as_uint(amax);
  int E;
  uint32_t mant;
  if ((ab >> 23) == 0u) {  // fp32 subnormal
    const int s = __clz(ab) - 8;
    mant = (ab << s) & 0x7FFFFFu;
    E = -126 - s;
  } else {
    E = (int)(ab >> 23) - 127;
    mant = ab & 0x7FFFFFu;
  }
  int X = E - 2 + (mant > 0x700000u ? 1 : 0);
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  const int ie = 127 - X;  // biased exponent of 2^-X, in [0, 254]
  const float inv = ie == 0 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)ie << 23);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e2m3_rne(v[i] * inv);
    const int bit = 6 * i, w = bit >> 5, sh = bit & 31;
    pk[w] |= c << sh;
    if (sh > 26) pk[w + 1] |= c >> (32 - sh);
  }
  sbyte = (uint32_t)(X + 127);
}

__global__ __launch_bounds__(kPT) void quant_x_kernel(const uint16_t* __restrict__ x, int nblk,
                                                      uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const int g = blockIdx.x * kPT + threadIdx.x;
  if (g >= nblk) return;
  const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)g * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = p[q];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      v[8 * q + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
  }
  uint32_t pk[6], sb;
  q6_block(v, pk, sb);
  uint2* dst = reinterpret_cast<uint2*>(xq + (size_t)g * 24);
  dst[0] = make_uint2(pk[0], pk[1]);
  dst[1] = make_uint2(pk[2], pk[3]);
  dst[2] = make_uint2(pk[4], pk[5]);
  xs[g] = (uint8_t)sb;
}

// ---- tile table --------------------------------------------------------------

struct TileTable {
  int nb;
  int total;
  int expert[kMaxExperts];
  int row0[kMaxExperts];
  int cnt[kMaxExperts];
  int tstart[kMaxExperts + 1];
};

// Non-empty buckets and the first tile index of each (tiles = ceil(cnt/BM) * ntw).
__device__ void build_tiles(const int32_t* __restrict__ offsets, int E, int ntw, TileTable& tt) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    constexpr int CH = kMaxExperts / 64;
    int off[CH + 1];
#pragma unroll
    for (int i = 0; i <= CH; ++i) {
      const int e = lane * CH + i;
      off[i] = offsets[e < E ? e : E];
    }
    int n = 0, nt = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = (lane * CH + i < E) ? off[i + 1] - off[i] : 0;
      if (c > 0) {
        ++n;
        nt += (c + BM - 1) / BM * ntw;
      }
    }
    int incl = n, tincl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64), ot = __shfl_up(tincl, d, 64);
      if (lane >= d) {
        incl += o;
        tincl += ot;
      }
    }
    int pos = incl - n, tpos = tincl - nt;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = lane * CH + i;
      const int c = (e < E) ? off[i + 1] - off[i] : 0;
      if (c > 0) {
        tt.expert[pos] = e;
        tt.row0[pos] = off[i];
        tt.cnt[pos] = c;
        tt.tstart[pos] = tpos;
        tpos += (c + BM - 1) / BM * ntw;
        ++pos;
      }
    }
    if (lane == 63) {
      tt.nb = incl;
      tt.total = tincl;
      tt.tstart[incl] = tincl;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int find_bucket(const TileTable& tt, int t) {
  int lo = 0, hi = tt.nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tt.tstart[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// XCD-aware walk: the tile list is cut into 8 contiguous ranges, and the
// workgroups on XCD x (blockIdx.x % 8 == x) take range x.
struct TileWalk {
  int next, end, step;
  __device__ TileWalk(int total) {
    const int xcd = blockIdx.x & 7, per = gridDim.x >> 3;
    const int lo = (int)((long)total * xcd / 8), hi = (int)((long)total * (xcd + 1) / 8);
    next = lo + (int)(blockIdx.x >> 3);
    end = hi;
    step = per;
  }
};

// ---- LDS buffers of the GEMMs -------------------------------------------------

struct GemmBuf {
  uint8_t a[BM * A_STRIDE];
  uint8_t b[128 * B_STRIDE];
  uint32_t as[BM];
  uint32_t bs[128];
};

struct GemmSmem {
  union {
    GemmBuf buf[2];
    float hbuf[BM * H_STRIDE];
  };
  int rowtok[BM];
};

// Registers holding one K chunk between its global loads and its LDS store.
struct ChunkRegs {
  uint4 a[3];   // 48 B: two 24-B blocks of one A row
  uint4 b[2];   // 32 B: two 16-B blocks of one B row
  uint32_t s;   // four scale bytes of one A row (tid < 128) or one B row (tid >= 128)
};

__device__ __forceinline__ void store_chunk(GemmBuf& d, const ChunkRegs& r, int tid) {
  const int row = tid >> 1, part = tid & 1;
  uint2* pa = reinterpret_cast<uint2*>(d.a + row * A_STRIDE + part * 48);
  pa[0] = make_uint2(r.a[0].x, r.a[0].y);
  pa[1] = make_uint2(r.a[0].z, r.a[0].w);
  pa[2] = make_uint2(r.a[1].x, r.a[1].y);
  pa[3] = make_uint2(r.a[1].z, r.a[1].w);
  pa[4] = make_uint2(r.a[2].x, r.a[2].y);
  pa[5] = make_uint2(r.a[2].z, r.a[2].w);
  uint4* pb = reinterpret_cast<uint4*>(d.b + row * B_STRIDE + part * 32);
  pb[0] = r.b[0];
  pb[1] = r.b[1];
  if (tid < 128) d.as[tid] = r.s; else d.bs[tid - 128] = r.s;
}

// 2 x 2 MFMA fragments of one wavefront over one K chunk: A fragments at LDS
// rows arow0 + 32f, B fragments at rows brow0 + bstep*g.
__device__ __forceinline__ void mma_chunk(const GemmBuf& d, f16v (&acc)[2][2], int arow0, int brow0, int bstep,
                                          int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int blk = 2 * s + h;
    i8v a[2], b[2];
    int sa[2], sb[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int row = arow0 + 32 * f + r32;
      const uint2* p = reinterpret_cast<const uint2*>(d.a + row * A_STRIDE + blk * 24);
      const uint2 q0 = p[0], q1 = p[1], q2 = p[2];
      a[f] = i8v{(int)q0.x, (int)q0.y, (int)q1.x, (int)q1.y, (int)q2.x, (int)q2.y, 0, 0};
      sa[f] = (int)((d.as[row] >> (8 * blk)) & 0xFFu);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int row = brow0 + bstep * g + r32;
      const uint4 q = *reinterpret_cast<const uint4*>(d.b + row * B_STRIDE + blk * 16);
      b[g] = i8v{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      sb[g] = (int)((d.bs[row] >> (8 * blk)) & 0xFFu);
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[f], b[g], acc[f][g], 2, 4, 0, sa[f], 0,
                                                                    sb[g]);
  }
}

// The K loop: two LDS buffers and a ring of three register sets, so the
// global loads of chunk c+3 are in flight while chunk c is multiplied and
// chunk c+1 is moved into LDS.
template <typename Load>
__device__ __forceinline__ void k_loop(GemmSmem& sm, f16v (&acc)[2][2], Load& load, int nchunks, int tid, int lane,
                                       int arow0, int brow0, int bstep) {
  ChunkRegs r0, r1, r2;
  load(0, r0);
  if (nchunks > 1) load(1, r1);
  if (nchunks > 2) load(2, r2);
  store_chunk(sm.buf[0], r0, tid);
  __syncthreads();
  auto step = [&](int c, ChunkRegs& next, ChunkRegs& spare) {
    if (c + 3 < nchunks) load(c + 3, spare);
    mma_chunk(sm.buf[c & 1], acc, arow0, brow0, bstep, lane);
    if (c + 1 < nchunks) store_chunk(sm.buf[(c + 1) & 1], next, tid);
    __syncthreads();
  };
  for (int c = 0; c < nchunks; c += 3) {
    step(c, r1, r0);
    if (c + 1 < nchunks) step(c + 1, r2, r1);
    if (c + 2 < nchunks) step(c + 2, r0, r2);
  }
}

// ---- P1: gate/up GEMM, SwiGLU and MXFP6 of h ----------------------------------

__global__ __launch_bounds__(kPT, 2) void gateup_mfma_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int k, int E, ExpertStore w,
    const int32_t* __restrict__ e2s, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair,
    uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ TileTable tt;
  __shared__ GemmSmem sm;
  const int H = w.H, I = w.I, NBH = H / 32, NBI = I / 32;
  const int ntw = I / 64;  // weight tiles: 64 gate rows + the same 64 up rows
  build_tiles(offsets, E, ntw, tt);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wm = wid >> 1, wn = wid & 1;
  const size_t arow_bytes = (size_t)NBH * 24, wrow_bytes = (size_t)H / 2;
  const int nchunks = H / BK;
  for (TileWalk tw(tt.total); tw.next < tw.end; tw.next += tw.step) {
    const int t = tw.next;
    const int b = find_bucket(tt, t);
    const int expert = tt.expert[b], row0 = tt.row0[b], cnt = tt.cnt[b];
    const int mtiles = (cnt + BM - 1) / BM, local = t - tt.tstart[b];
    const int ntile = local / mtiles, mtile = local - ntile * mtiles;
    const int slot = e2s ? e2s[expert] : expert;
    if (slot < 0 || slot >= w.num_slots) continue;  // the down GEMM writes zero rows
    const int m0 = mtile * BM, n0 = ntile * 64;
    const int mrows = min(BM, cnt - m0);
    if (tid < BM) sm.rowtok[tid] = tid < mrows ? sorted_pair[row0 + m0 + tid] / k : -1;
    __syncthreads();
    // this thread's load sources
    const int lrow = tid >> 1, part = tid & 1;
    const int tok = sm.rowtok[lrow];
    const uint8_t* asrc = tok >= 0 ? xq + (size_t)tok * arow_bytes + part * 48 : nullptr;
    const int wmat = lrow >> 6, wn_row = n0 + (lrow & 63);
    const uint8_t* bsrc = (wmat ? w.wu : w.wg) + ((size_t)slot * I + wn_row) * wrow_bytes + part * 32;
    const uint8_t* ssrc;
    if (tid < BM) {
      const int st = sm.rowtok[tid];
      ssrc = st >= 0 ? xs + (size_t)st * NBH : nullptr;
    } else {
      const int r = tid - BM;
      ssrc = (r >> 6 ? w.su : w.sg) + ((size_t)slot * I + n0 + (r & 63)) * NBH;
    }
    auto load = [&](int c, ChunkRegs& r) {
      if (asrc) {
        const uint4* p = reinterpret_cast<const uint4*>(asrc + (size_t)c * 96);
        r.a[0] = p[0];
        r.a[1] = p[1];
        r.a[2] = p[2];
      } else {
        r.a[0] = r.a[1] = r.a[2] = make_uint4(0, 0, 0, 0);
      }
      const uint4* q = reinterpret_cast<const uint4*>(bsrc + (size_t)c * 64);
      r.b[0] = q[0];
      r.b[1] = q[1];
      r.s = ssrc ? *reinterpret_cast<const uint32_t*>(ssrc + c * 4) : 0x7F7F7F7Fu;
    };
    f16v acc[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[f][g] = f16v{};
    k_loop(sm, acc, load, nchunks, tid, lane, 64 * wm, 32 * wn, 64);  // B: gate rows 32wn.., up 64+32wn..
    // h = silu(g) * u into the staging buffer, then MXFP6 per (row, 32-block)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 64 * wm + 32 * f + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        const int col = 32 * wn + (lane & 31);
        sm.hbuf[row * H_STRIDE + col] = swiglu_f32(acc[f][0][i], acc[f][1][i]);
      }
    }
    __syncthreads();
    {
      const int row = tid >> 1, blk = tid & 1;
      if (row < mrows) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = sm.hbuf[row * H_STRIDE + 32 * blk + i];
        uint32_t pk[6], sb;
        q6_block(v, pk, sb);
        const size_t grow = (size_t)(row0 + m0 + row);
        const int gblk = n0 / 32 + blk;
        uint2* dst = reinterpret_cast<uint2*>(hq + grow * NBI * 24 + (size_t)gblk * 24);
        dst[0] = make_uint2(pk[0], pk[1]);
        dst[1] = make_uint2(pk[2], pk[3]);
        dst[2] = make_uint2(pk[4], pk[5]);
        hs[grow * NBI + gblk] = (uint8_t)sb;
      }
    }
    __syncthreads();
  }
}

// ---- P2: down GEMM -> y_pair ---------------------------------------------------

__global__ __launch_bounds__(kPT, 2) void down_mfma_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, int E, ExpertStore w,
    const int32_t* __restrict__ e2s, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair,
    float* __restrict__ y) {
  __shared__ TileTable tt;
  __shared__ GemmSmem sm;
  const int H = w.H, I = w.I, NBI = I / 32;
  const int ntw = H / 128;
  build_tiles(offsets, E, ntw, tt);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wm = wid >> 1, wn = wid & 1;
  const size_t arow_bytes = (size_t)NBI * 24, wrow_bytes = (size_t)I / 2;
  const int nchunks = I / BK;
  for (TileWalk tw(tt.total); tw.next < tw.end; tw.next += tw.step) {
    const int t = tw.next;
    const int b = find_bucket(tt, t);
    const int expert = tt.expert[b], row0 = tt.row0[b], cnt = tt.cnt[b];
    const int mtiles = (cnt + BM - 1) / BM, local = t - tt.tstart[b];
    const int ntile = local / mtiles, mtile = local - ntile * mtiles;
    const int slot = e2s ? e2s[expert] : expert;
    const int m0 = mtile * BM, n0 = ntile * 128;
    const int mrows = min(BM, cnt - m0);
    if (tid < BM) sm.rowtok[tid] = tid < mrows ? sorted_pair[row0 + m0 + tid] : -1;
    __syncthreads();
    if (slot < 0 || slot >= w.num_slots) {
      for (int i = tid; i < mrows * 128; i += kPT) {
        const int row = i >> 7, col = i & 127;
        y[(size_t)sm.rowtok[row] * H + n0 + col] = 0.f;
      }
      __syncthreads();
      continue;
    }
    const int lrow = tid >> 1, part = tid & 1;
    const uint8_t* asrc = lrow < mrows ? hq + (size_t)(row0 + m0 + lrow) * arow_bytes + part * 48 : nullptr;
    const uint8_t* bsrc = w.wd + ((size_t)slot * H + n0 + lrow) * wrow_bytes + part * 32;
    const uint8_t* ssrc;
    if (tid < BM)
      ssrc = tid < mrows ? hs + (size_t)(row0 + m0 + tid) * NBI : nullptr;
    else
      ssrc = w.sd + ((size_t)slot * H + n0 + (tid - BM)) * NBI;
    auto load = [&](int c, ChunkRegs& r) {
      if (asrc) {
        const uint4* p = reinterpret_cast<const uint4*>(asrc + (size_t)c * 96);
        r.a[0] = p[0];
        r.a[1] = p[1];
        r.a[2] = p[2];
      } else {
        r.a[0] = r.a[1] = r.a[2] = make_uint4(0, 0, 0, 0);
      }
      const uint4* q = reinterpret_cast<const uint4*>(bsrc + (size_t)c * 64);
      r.b[0] = q[0];
      r.b[1] = q[1];
      r.s = ssrc ? *reinterpret_cast<const uint32_t*>(ssrc + c * 4) : 0x7F7F7F7Fu;
    };
    f16v acc[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[f][g] = f16v{};
    k_loop(sm, acc, load, nchunks, tid, lane, 64 * wm, 64 * wn, 32);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 64 * wm + 32 * f + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          if (row < mrows) {
            const int col = n0 + 64 * wn + 32 * g + (lane & 31);
            y[(size_t)sm.rowtok[row] * H + col] = acc[f][g][i];
          }
        }
      }
    }
    __syncthreads();
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t prefill_workspace_bytes(int T, int k, int H, int I) {
  const size_t P = (size_t)T * k;
  return align256((size_t)T * H / 32 * 24) + align256((size_t)T * H / 32) + align256(P * I / 32 * 24) +
         align256(P * I / 32);
}

hipError_t launch_prefill(const uint16_t* x, int T, int k, int E, const ExpertStore& w, const int32_t* e2s,
                          const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws,
                          hipStream_t s) {
  const int H = w.H, I = w.I;
  if (H % 128 != 0 || I % 128 != 0) return hipErrorInvalidValue;
  const size_t P = (size_t)T * k;
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint8_t* xq = base;
  uint8_t* xs = xq + align256((size_t)T * H / 32 * 24);
  uint8_t* hq = xs + align256((size_t)T * H / 32);
  uint8_t* hs = hq + align256(P * I / 32 * 24);
  const int nblk = T * (H / 32);
  hipLaunchKernelGGL(quant_x_kernel, dim3((nblk + kPT - 1) / kPT), dim3(kPT), 0, s, x, nblk, xq, xs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gateup_mfma_kernel, dim3(kGrid), dim3(kPT), 0, s, xq, xs, k, E, w, e2s, offsets, sorted_pair,
                     hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(down_mfma_kernel, dim3(kGrid), dim3(kPT), 0, s, hq, hs, E, w, e2s, offsets, sorted_pair,
                     y_pair);
  return hipGetLastError();
}

}  // namespace moe
