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
//   P0  quant_x:  x bf16 [T][H] -> MXFP6 blocks per token (scratch)
//       sort_x:   -> xq, xs in bucket-sorted rows, chunk-major (one 48-B record per
//                 row, 128-K chunk and K-half; see q6_offset)
//   plan:         bucket offsets -> flat tile lists of both GEMMs
//   P1  gateup:   per tile: g = W_gate.x, u = W_up.x (MFMA, fp32),
//                 h = silu(g)*u, h -> MXFP6 into hq/hs (sorted-row order)
//   P2  down:     per tile: y = W_down.h (MFMA, fp32) -> y_pair row p
//
// Buckets of more than 32 rows run as GEMM tiles of 128 bucket rows x 512
// weight rows over all of K (the grouped GEMM core below); smaller buckets,
// whose experts are read once for a handful of rows, as a weight stream (the
// streaming path).  The tile workgroups are persistent: the tile list (bucket,
// weight tile, row tile -- row tiles of one weight tile adjacent, so they
// share that weight tile in L2) is split into eight contiguous ranges, one
// per XCD.
//
// The weights come either from the row-major expert store (each load covers
// 8 rows x 128 B and is reordered through LDS into operand order) or from a
// copy of the experts in operand order (pack_weights_kernel, made once when
// the experts are loaded), from which each K-step's operand is one
// contiguous 1 KB load straight into the MFMA's register.  Both give the
// same bytes to the same MFMAs in the same order.
#include "common.cuh"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPT = 256;  // threads per workgroup


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

// Scale of a block whose largest magnitude is amax > 0: block exponent
// X = floor(log2 amax) - 2 (+1 when the significand of amax exceeds 1.875),
// clamped to [-127, 127].  Returns the scale byte X + 127; inv = 2^-X.
__device__ __forceinline__ uint32_t q6_scale(float amax, float& inv) {
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
  inv = ie == 0 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)ie << 23);
  return (uint32_t)(X + 127);
}

// One 32-element block -> 24 packed bytes (code i at bits 6i..6i+5) + scale
// byte (q6_scale); amax == 0 gives scale 0, codes 0.
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
  float inv;
  sbyte = q6_scale(amax, inv);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e2m3_rne(v[i] * inv);
    const int bit = 6 * i, w = bit >> 5, sh = bit & 31;
    pk[w] |= c << sh;
    if (sh > 26) pk[w + 1] |= c >> (32 - sh);
  }
}

// MXFP6 rows in the layout the GEMMs read.  Row p is a sorted (bucket-order)
// row; K runs in chunks of 128 (blocks 4c..4c+3).  For chunk c and K-half
// h (blocks h and 2+h: the lane's operand for the chunk's two MFMA K-steps)
// the rows' 48-byte records are contiguous:
//   codes: [c][h][p][48 B] (block h, then block 2+h, 24 B each)
//   x scales: [c][p] words (the scale bytes of blocks 4c..4c+3)
// so a tile's chunk is two contiguous runs of 48-byte records, in the order
// the LDS stage holds them.
__device__ __forceinline__ size_t q6_offset(int p, int b, int P) {
  const int c = b >> 2, bb = b & 3;
  return ((size_t)(2 * c + (bb & 1)) * P + p) * 48 + (size_t)(bb >> 1) * 24;
}

// Each token's x once: one thread per 32-block, token-major codes [T][H/32][24 B]
// and scale bytes [T][H/32].
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

// The token-major blocks copied into the sorted chunk-major layout.  One
// wavefront per (chunk c, 64 consecutive sorted rows): each lane reads its
// row's 96 B of the chunk (the four blocks of its token) into the wavefront's
// LDS area as the row's two 48-byte records, then the wavefront writes each
// K-half's 64 records, 3 KB contiguous in xq, with three 16-byte stores per
// lane (every store instruction one contiguous 1 KB), and the chunk's scale
// words.  Only the rows that the bucketing filled are written: sorted rows at
// or past offsets[E] (pairs whose expert id was out of range are in no
// bucket) hold no pair index, and a pair index outside [0, T*k) is skipped
// as well.
__global__ __launch_bounds__(kPT) void sort_x_kernel(const uint8_t* __restrict__ xq_t,
                                                     const uint8_t* __restrict__ xs_t, int H, int k, int P,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     const int32_t* __restrict__ sorted_pair,
                                                     uint8_t* __restrict__ xq, uint32_t* __restrict__ xs) {
  __shared__ __attribute__((aligned(16))) uint8_t rec[kPT / 64][2][64 * 48];
  __shared__ uint8_t ok[kPT / 64][64];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = H / 128, ngrp = (P + 63) / 64, gw = blockIdx.x * (kPT / 64) + wid;
  if (gw >= nch * ngrp) return;
  const int c = gw / ngrp, p0 = (gw - c * ngrp) * 64, p = p0 + lane, nvalid = offsets[E];
  if (p0 >= nvalid) return;
  const int pair = p < nvalid ? sorted_pair[p] : -1;
  const bool valid = pair >= 0 && pair < P;
  const size_t t = valid ? (size_t)(pair / k) : 0;
  uint32_t u[24] = {};  // block b of the chunk = u[6b .. 6b+5]
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(xq_t + (t * (H / 32) + 4 * c) * 24);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const uint4 v = src[i];
      u[4 * i] = v.x, u[4 * i + 1] = v.y, u[4 * i + 2] = v.z, u[4 * i + 3] = v.w;
    }
    xs[(size_t)c * P + p] = *reinterpret_cast<const uint32_t*>(xs_t + t * (H / 32) + 4 * c);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {  // record of K-half h: block h, then block 2+h
    uint32_t* r = reinterpret_cast<uint32_t*>(rec[wid][h] + lane * 48);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      r[i] = u[6 * h + i];
      r[6 + i] = u[6 * (2 + h) + i];
    }
  }
  ok[wid][lane] = valid ? 1 : 0;
  // other lanes' records are read next: wavefront-scope fences keep the
  // compiler's order (a wavefront's LDS accesses complete in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint8_t* dst = xq + ((size_t)(2 * c + h) * P + p0) * 48;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int off = 1024 * j + 16 * lane, r = off / 48;  // a 16-byte piece lies in one record
      if (p0 + r < nvalid && ok[wid][r])
        *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(rec[wid][h] + off);
    }
  }
}

// ---- tile plan -----------------------------------------------------------------
//
// One small kernel turns the bucket offsets into two flat tile lists, one per
// GEMM, ordered expert by expert, then by weight tile, then by row tile, so
// the row tiles that share a weight tile are neighbours (and run at the same
// time on one XCD, sharing that weight tile in its L2).  Every workgroup
// computes the per-expert tile prefix (a few thousand LDS operations) and
// writes its grid-stride share of the tiles; workgroup 0 writes the
// small-bucket list and the counts.

constexpr int BM = 128;            // bucket rows per tile
constexpr int KC = 128;            // K per chunk (4 scale blocks, 2 MFMA K-steps)
constexpr int GU_N = 256;          // gate/up tile: 256 h columns = 256 gate + 256 up weight rows
constexpr int DN_N = 512;          // down tile: 512 output columns
constexpr int kGrid = 256;         // persistent workgroups (one per CU: the LDS holds one)

constexpr int SK_MAX = 32;  // buckets with at most this many rows take the streaming kernels
constexpr int kPlanGrid = 32;  // workgroups of the plan kernel

struct SkBucket {
  int32_t row0;  // first sorted row
  int32_t cnt;   // rows (1..SK_MAX)
  int32_t slot;  // storage slot of the expert, -1 if it has none
  int32_t pad;
};

struct TileDesc {
  int32_t row0;   // first sorted row of the tile
  int32_t mrows;  // rows in the tile (1..BM)
  int32_t slot;   // storage slot of the expert, -1 if it has none
  int32_t ntile;  // weight tile
};

// Exclusive prefix sum over the workgroup of one value per thread; *total gets the sum.
__device__ int block_exclusive_sum(int v, int* part, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) part[wid] = incl;
  __syncthreads();
  int base = 0, sum = 0;
  for (int w = 0; w < kPT / 64; ++w) {
    if (w < wid) base += part[w];
    sum += part[w];
  }
  *total = sum;
  return base + incl - v;
}

__global__ __launch_bounds__(kPT) void plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                   const int32_t* __restrict__ e2s, int num_slots, int ntw_gu,
                                                   int ntw_dn, const uint8_t* __restrict__ run,
                                                   TileDesc* __restrict__ gu, TileDesc* __restrict__ dn,
                                                   SkBucket* __restrict__ sbk, int32_t* __restrict__ counts) {
  __shared__ int mstart[kMaxExperts + 1];
  __shared__ int offs[kMaxExperts + 1];  // the bucket offsets and slots, read once: the tile loop
  __shared__ int slots[kMaxExperts];     // below touches them once per tile
  __shared__ int part[kPT / 64];
  const int tid = threadIdx.x;
  for (int e = tid; e <= kMaxExperts; e += kPT) {
    offs[e] = offsets[e < E ? e : E];
    if (e < kMaxExperts) {
      int slot = e < E ? (e2s ? e2s[e] : e) : -1;
      slots[e] = (slot < 0 || slot >= num_slots) ? -1 : slot;
    }
  }
  __syncthreads();
  constexpr int PER = kMaxExperts / kPT;  // experts per thread
  int mt[PER], small[PER];
  int msum = 0, ssum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    // experts outside the run mask get no work: their rows are left untouched
    const int c = (e < E && (run == nullptr || run[e] != 0)) ? offs[e + 1] - offs[e] : 0;
    small[i] = (c >= 1 && c <= SK_MAX) ? 1 : 0;
    mt[i] = small[i] ? 0 : (c + BM - 1) / BM;
    msum += mt[i];
    ssum += small[i];
  }
  int nm, ns;
  int mrun = block_exclusive_sum(msum, part, &nm);
  int srun = block_exclusive_sum(ssum, part, &ns);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    mstart[e] = mrun;
    mrun += mt[i];
    if (small[i] && blockIdx.x == 0) {
      SkBucket b;
      b.row0 = offs[e];
      b.cnt = offs[e + 1] - offs[e];
      b.slot = slots[e];
      b.pad = 0;
      sbk[srun++] = b;
    }
  }
  if (tid == kPT - 1) mstart[kMaxExperts] = mrun;
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    const int ntw = pass ? ntw_dn : ntw_gu;
    TileDesc* out = pass ? dn : gu;
    const int total = nm * ntw;
    for (int t = blockIdx.x * kPT + tid; t < total; t += gridDim.x * kPT) {
      // expert e with mstart[e]*ntw <= t < mstart[e+1]*ntw (experts without row tiles have equal bounds)
      int lo = 0, hi = kMaxExperts - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mstart[mid] * ntw <= t) lo = mid; else hi = mid - 1;
      }
      const int e = lo;
      const int mtiles = mstart[e + 1] - mstart[e];
      const int local = t - mstart[e] * ntw;
      const int ntile = local / mtiles, mtile = local - ntile * mtiles;
      const int c = offs[e + 1] - offs[e];
      TileDesc d;
      d.row0 = offs[e] + mtile * BM;
      d.mrows = min(BM, c - mtile * BM);
      d.slot = slots[e];
      d.ntile = ntile;
      out[t] = d;
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    counts[0] = nm * ntw_gu;
    counts[1] = nm * ntw_dn;
    counts[2] = ns;
  }
}

// XCD-aware walk: the tile list is cut into 8 contiguous ranges, and the
// workgroups on XCD x (blockIdx.x % 8 == x) take range x in turn.
struct TileWalk {
  int next, end, step;
  __device__ TileWalk(int total) {
    const int xcd = blockIdx.x & 7, per = gridDim.x >> 3;
    next = (int)((long)total * xcd / 8) + (int)(blockIdx.x >> 3);
    end = (int)((long)total * (xcd + 1) / 8);
    step = per;
  }
};


constexpr uint32_t kOpenRange = 0x7FFFFFF0u;  // range of the activation buffers (offsets < 2^31)

// ---- the grouped GEMM core ---------------------------------------------------------
//
// A tile is BM = 128 bucket rows x 8 * WN = 512 weight rows over all of K, in
// chunks of 128 (four 32-blocks, two K-steps of V_MFMA_SCALE_F32_32X32X64),
// processed a pair of chunks at a time by eight wavefronts, two per SIMD.
// Each wavefront owns WN = 64 weight rows (two 32-row fragments) and all 128
// bucket rows (four fragments): 8 MFMAs per K-step into 4 x 2 accumulators of
// 16 fp32 per lane (128 AGPRs), which leaves 128 VGPRs for everything else.
//
// Loads.  What a load costs is the number of distinct weight rows it touches
// and what a CU keeps in flight, not its bytes: a load over the 32 rows of an
// MFMA operand streams at ~38 GB/s per CU even from L2, one over 8 rows x
// 128 B at up to ~100, and once the rows live beyond L2 the rate grows with
// the loads in flight (two wavefronts per SIMD, 8-row loads: ~80 GB/s per CU
// against ~30 for one).  So each wavefront loads its weight rows for a chunk
// pair as 8 rows x 128 B per load (lane l: row 8 j + l / 8, bytes 16 (l % 8)
// of the pair), writes them into a private LDS area and reads them back in
// operand order; the next pair's loads go out as soon as the registers are
// written.  The weights' scale bytes go to registers two pairs at a time: a
// scale load touches one line per row whatever its width, so each lane loads
// one pair's 8 bytes of its row (lane l: pair l / 32) and swaps them with its
// partner l ^ 32, half the loads and lines of one load per pair (removing
// the scale loads altogether sped the GEMMs up by 10-14%).  The activations are shared by the eight wavefronts: each
// chunk's 128 records are copied from memory into one of four LDS stages by
// the buffer unit (buffer_load ... lds, no registers; two copies of 1 KB per
// wavefront), a pair ahead, and read from there by every
// wavefront; their scale words come from an LDS table filled once per window
// of TWIN chunks.  One barrier per pair: before it, each wavefront waits for
// its own copies of the next pair; the stages they fill were last read before
// the previous one.
//
// The gate/up GEMM puts the weights in the MFMA's first operand, so an
// accumulator holds one bucket row per lane (row l % 32 of its fragment) and
// 16 weight rows per register set, 8 (r / 4) + 4 (l / 32) + r % 4 of the
// fragment's 32: the gate and up rows of a wavefront are the same 32 h
// columns, half of each MXFP6 block in one lane and half in its partner l ^ 32,
// so the epilogue needs one lane swap per block and no LDS.  The down GEMM
// puts the activations first, so a lane holds one output column of 16 rows
// and a store writes 32 consecutive columns of a y_pair row.

// A copy of v that the compiler cannot see through: per-lane index arithmetic
// derived from it is recomputed where it is used instead of being hoisted out
// of the persistent tile loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

constexpr int kTilePT = 512;        // threads of a tile workgroup: eight wavefronts
constexpr int WN = 64;              // weight rows per wavefront (two fragments)
constexpr int A_HS = BM * 48 + 64;  // LDS bytes per K-half region of an A stage
constexpr int A_STAGE = 2 * A_HS;   // LDS bytes per A stage (one chunk)
constexpr int TWIN = 40;            // scale-table window in chunks (even: whole pairs)
constexpr int B_FRAG = 32 * 128;    // LDS bytes of one fragment's pair in operand order
constexpr int B_SCR = 2 * B_FRAG;   // a wavefront's weight reorder area

// Table word of row r (of 128) and chunk wd of the window, chunk-major: a
// lane's words of rows r32 + 32 f, f = 0..3, are one 16-byte read.  One chunk
// column more than the window, read (never used) after its last chunk.
__device__ __forceinline__ int cf_index(int row, int wd) { return (32 * wd + (row & 31)) * 4 + (row >> 5); }
constexpr int TAB_WORDS = (TWIN + 1) * 128;

struct TileTables {
  uint32_t sca[TAB_WORDS];  // activation scale words of the tile's 128 rows
};

// Words [cw0, cw0 + WIN) of ROWS table rows from a chunk-major word array
// ([chunk][row], row stride 1 word, P rows per chunk): consecutive threads
// read consecutive rows of one chunk.  Rows at or past nrows read zeros.
template <int ROWS, int NT, int WIN, int STRIDE>
struct ScaleCols {
  static constexpr int N = ROWS * WIN / NT;
  static_assert(ROWS * WIN % NT == 0 && WIN < STRIDE, "table split");
  uint32_t v[N];
  __device__ __forceinline__ void issue(rsrc_t r, int cw0, int t, int row0, int nrows, int P) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = t + NT * i, wd = idx / ROWS, row = idx - wd * ROWS;
      v[i] = bload4(r, row < nrows ? ((uint32_t)(cw0 + wd) * (uint32_t)P + (uint32_t)(row0 + row)) * 4u : kOob);
    }
  }
  __device__ __forceinline__ void store(uint32_t* tab, int t) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = t + NT * i, wd = idx / ROWS, row = idx - wd * ROWS;
      tab[row * STRIDE + wd] = v[i];
    }
  }
  // The same words in the chunk-major order of the tile tables (128 rows).
  __device__ __forceinline__ void store_cf(uint32_t* tab, int t) const {
    static_assert(ROWS == 128, "four 32-row fragments");
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = t + NT * i, wd = idx / ROWS, row = idx - wd * ROWS;
      tab[cf_index(row, wd)] = v[i];
    }
  }
};

// The activation records of a tile's chunk: two runs (K-half 0, then 1) of 128
// rows x 48 B, 12 KB, copied into an LDS stage as 12 pieces of 1 KB (64 lanes x
// 16 B; a 12-byte copy into LDS leaves a lane 16 bytes).  Wavefront w copies
// pieces w and w + 8; wavefronts 4-7, which have no second piece, copy their
// first one again (the same bytes to the same place), so every wavefront
// issues two copies per chunk.  Memory and the stage hold the runs in the same
// order; the stage pads each run by 64 B.  Rows past the bucket read other
// buckets' records (their outputs are never stored and their scale words are
// zero); past the array's end they read zeros.
struct ACopy {
  rsrc_t rc;
  uint32_t vc[2];    // the lane's 16 B of each piece in chunk 0
  uint32_t cstride;  // bytes per chunk: both K-halves of all P rows
  int lo[2];         // LDS offset of each piece in a stage (the same in every lane)
  __device__ __forceinline__ void init(const uint8_t* base, uint32_t bytes, int wid, int lane, int row0, int P) {
    rc = make_rsrc(base, bytes);
    cstride = 96u * (uint32_t)P;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = j == 1 && wid + 8 < 12 ? wid + 8 : wid, h = i / 6, q = i - 6 * h;  // 6 pieces per run
      vc[j] = ((uint32_t)h * (uint32_t)P + (uint32_t)row0) * 48u + (uint32_t)q * 1024u + (uint32_t)lane * 16u;
      lo[j] = h * A_HS + q * 1024;
    }
  }
  // Chunk c into stage st; c < 0 copies nothing useful (zeros).
  __device__ __forceinline__ void copy(uint8_t* st, int c) const {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)(st + lo[j]), 16,
                                               c < 0 ? kOob : vc[j] + (uint32_t)c * cstride, 0, 0, 0);
  }
};

// The lane's activation operand of K-step S of fragment f: 24 bytes at offset
// 24 S of the 48-byte record of row 32 f + r32 in K-half h (blocks 4c + h and
// 4c + 2 + h).
template <int S>
__device__ __forceinline__ i8v read_afrag(const uint8_t* st, int f, int r32, int h) {
  const uint8_t* p = st + h * A_HS + (32 * f + r32) * 48 + 24 * S;
  if (S == 0) {
    const uint4_t a = *reinterpret_cast<const uint4_t*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 16);
    return i8v{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, 0, 0};
  } else {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint4_t b = *reinterpret_cast<const uint4_t*>(p + 8);
    return i8v{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0};
  }
}

// One wavefront's weight rows for a chunk pair as loaded: fragment g's 32
// rows x 128 B in four loads of 8 rows (q[g][j]: rows 8 j + l / 8, bytes
// 16 (l % 8)).
struct BRaw {
  uint4_t q[2][4];
};

struct BSrc {
  rsrc_t rc[2], rs[2];  // codes and scales of the matrix holding each fragment
  uint32_t vc[2];       // the lane's code bytes in chunk 0: row l / 8 of the fragment, + 16 (l % 8)
  uint32_t vs[2];       // the lane's scale bytes in group 0: row l % 32 of the fragment, pair l / 32
  uint32_t row8;        // bytes from a weight row to the row 8 below
  // Codes of fragment g of the pair starting at chunk c (even); c < 0 loads zeros.
  // Past the row's last chunk the bytes belong to the next row (never used).
  __device__ __forceinline__ void load(int g, int c, BRaw& r) const {
    const bool z = c < 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.q[g][j] = bload16(rc[g], z ? kOob : vc[g] + (uint32_t)j * row8 + (uint32_t)c * 64u);
  }
  // Scale bytes of fragment g for the two pairs starting at chunk c (c % 4 == 0):
  // the lane gets those of pair l / 32 (8 bytes); c < 0 loads zeros.
  __device__ __forceinline__ uint2 load_scales(int g, int c) const {
    return bload8(rs[g], c < 0 ? kOob : vs[g] + (uint32_t)c * 4u);
  }
};

// A lane's weight scale words of the two pairs of a group, from the 8 bytes of
// its row that it loaded (pair h = l / 32) and the 8 its partner lane l ^ 32
// loaded: word p holds bytes h and 2 + h of chunk 2p's scale word, then of
// chunk 2p + 1's, so byte S is the scale of K-step S of pair p.
__device__ __forceinline__ void group_words(const uint2& own, int h, uint32_t (&pk)[2]) {
  const auto x0 = __builtin_amdgcn_permlane32_swap(own.x, own.x, false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(own.y, own.y, false, false);
  const uint32_t o0 = h ? x0[0] : x0[1], o1 = h ? x1[0] : x1[1];  // the partner's pair
  const uint32_t sel = 0x06040200u + 0x01010101u * (uint32_t)h;
  const uint32_t mine = __builtin_amdgcn_perm(own.y, own.x, sel), other = __builtin_amdgcn_perm(o1, o0, sel);
  pk[0] = h ? other : mine;
  pk[1] = h ? mine : other;
}

__device__ __forceinline__ i8v bop(const uint4_t& q) { return i8v{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0}; }

// s_waitcnt with only the vector-memory count: every vector memory operation
// but the n most recent has completed (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt with only the LDS count: this wavefront's LDS operations have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Workgroup barrier without the release fence of __syncthreads(), which would
// wait for every copy into LDS in flight: each caller first waits for what the
// other wavefronts will read.  The acquire fence (no instructions at workgroup
// scope) keeps the compiler from moving later LDS reads above the barrier.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Vector memory operations of a pair: four LDS copies (two chunks), then per
// weight fragment four code loads (and a scale load in a group's first pair).
constexpr int kPairCodeVm = 2 * 4;
// The same with operand-order weights: per fragment four operand loads and a scale load.
constexpr int kPairPkVm = 2 * 5;

// A lane's scale words of chunk wd (rows r32 + 32 f of the table), shifted so
// that byte 0 is the scale of its block 4c + h (K-step 0) and byte 2 that of
// block 4c + 2 + h (K-step 1).
__device__ __forceinline__ uint4_t scale_words(const uint32_t* tab, int wd, int r32, int h) {
  const uint4_t w = *reinterpret_cast<const uint4_t*>(tab + (32 * wd + r32) * 4);
  const int s = 8 * h;
  return uint4_t{w.x >> s, w.y >> s, w.z >> s, w.w >> s};
}

__device__ __forceinline__ int word(const uint4_t& w, int f) {
  return (int)(f == 0 ? w.x : f == 1 ? w.y : f == 2 ? w.z : w.w);
}

// One MFMA of the tile: weights W (fp4, scale byte opsel of sw) against
// activations A (fp6, scale byte opsel of sa).  WFIRST: the weights are the
// first operand (accumulators hold one bucket row per lane) or the second
// (one output column per lane).
template <bool WFIRST, int OW, int OA>
__device__ __forceinline__ f16v tile_mfma(const i8v& W, const i8v& A, const f16v& c, int sw, int sa) {
  if (WFIRST) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(W, A, c, 4, 2, OW, sw, OA, sa);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, W, c, 2, 4, OA, sa, OW, sw);
}

// Pair q of a window (chunks c0 = cw0 + 2q and c0 + 1, in stages 2 PJ and
// 2 PJ + 1; raw and ws hold its weights as loaded).  The copies of the next
// pair go out first, into the other two stages; then the fragments' rows are
// written into the wavefront's LDS area in operand order (K-step S at
// S * 1024, lane t's 16 B at slot t ^ 2 S, so both the writes and the reads
// stay within two LDS banks per slot) and the registers reloaded with the
// next pair; then the four K-steps: the activation fragments and the two
// weight operands are read, 8 MFMAs.  run0 / run1: chunk c0 / c0 + 1 exists.
template <int PJ, bool WFIRST>
__device__ __forceinline__ void tile_pair(const TileTables& tb, uint8_t* const (&st)[4], uint8_t* scr,
                                          const ACopy& as, const BSrc& bs, BRaw& raw, uint2 (&sraw)[2],
                                          uint32_t (&pk)[2][2], f16v (&acc)[4][2], int cw0, int last, int q,
                                          int lane, int r32, int h, bool run0, bool run1) {
  const int c0 = cw0 + 2 * q, n0 = c0 + 2;
  if (PJ == 0) {
#pragma unroll
    for (int g = 0; g < 2; ++g) group_words(sraw[g], h, pk[g]);
  }
  as.copy(st[2 - 2 * PJ], n0 <= last ? n0 : -1);
  as.copy(st[3 - 2 * PJ], n0 + 1 <= last ? n0 + 1 : -1);
  __builtin_amdgcn_sched_barrier(0);
  {
    const int r8 = lane >> 3, s = lane & 7, S = s >> 1, hh = s & 1;
    uint8_t* wr = scr + S * 1024 + ((r8 ^ (2 * S)) + 32 * hh) * 16;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4_t*>(wr + g * B_FRAG + j * 128) = raw.q[g][j];
  }
  __builtin_amdgcn_sched_barrier(0);
  if (PJ == 0) {
    const int cn = c0 + 4;  // the next group
#pragma unroll
    for (int g = 0; g < 2; ++g) sraw[g] = bs.load_scales(g, cn <= last ? cn : -1);
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) bs.load(g, n0 <= last ? n0 : -1, raw);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int S = 0; S < 4; ++S) {
    if (S < 2 ? !run0 : !run1) continue;
    const uint8_t* sta = st[2 * PJ + (S >> 1)];
    const uint4_t sa = scale_words(tb.sca, c0 + (S >> 1) - cw0, r32, h);
    i8v a[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) a[f] = (S & 1) ? read_afrag<1>(sta, f, r32, h) : read_afrag<0>(sta, f, r32, h);
    uint4_t b[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
      b[g] = *reinterpret_cast<const uint4_t*>(scr + g * B_FRAG + S * 1024 + ((lane ^ (2 * S)) * 16));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int sw = (int)pk[g][PJ];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (S == 0) acc[f][g] = tile_mfma<WFIRST, 0, 0>(bop(b[g]), a[f], acc[f][g], sw, word(sa, f));
        if (S == 1) acc[f][g] = tile_mfma<WFIRST, 1, 2>(bop(b[g]), a[f], acc[f][g], sw, word(sa, f));
        if (S == 2) acc[f][g] = tile_mfma<WFIRST, 2, 0>(bop(b[g]), a[f], acc[f][g], sw, word(sa, f));
        if (S == 3) acc[f][g] = tile_mfma<WFIRST, 3, 2>(bop(b[g]), a[f], acc[f][g], sw, word(sa, f));
      }
    }
  }
  if (PJ == 0) wait_vm<kPairCodeVm + 2>();  // this wavefront's copies of the next pair are done
  else wait_vm<kPairCodeVm>();
  wg_barrier();
}

// All K of one tile.  The first pair's copies go out before the window's
// scale table and its weight loads after; the table's stores wait for every
// load before them, so the copies are done, and the barrier publishes the
// table and the first stages.  tables(cw0) issues and stores the scale table
// of a window.
template <bool WFIRST, typename Tables>
__device__ __forceinline__ void tile_k_loop(TileTables& tb, uint8_t* const (&st)[4], uint8_t* scr,
                                            f16v (&acc)[4][2], const ACopy& as, const BSrc& bs, int nch, int tid,
                                            Tables tables) {
  const int lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  for (int cw0 = 0; cw0 < nch; cw0 += TWIN) {
    const int last = min(cw0 + TWIN, nch) - 1;
    if (cw0 > 0) wg_barrier();  // every wavefront is done with the previous window
    as.copy(st[0], cw0);
    as.copy(st[1], cw0 + 1 <= last ? cw0 + 1 : -1);
    tables(cw0);
    __builtin_amdgcn_sched_barrier(0);
    BRaw raw;
    uint2 sraw[2];
    uint32_t pk[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g) sraw[g] = bs.load_scales(g, cw0);
#pragma unroll
    for (int g = 0; g < 2; ++g) bs.load(g, cw0, raw);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kPairCodeVm>();  // all but the code loads just issued
    wait_lgkm0();            // the table stores
    wg_barrier();
    for (int q = 0; cw0 + 2 * q <= last; q += 2) {
      const int c = cw0 + 2 * q;
      tile_pair<0, WFIRST>(tb, st, scr, as, bs, raw, sraw, pk, acc, cw0, last, q, lane, r32, h, true, c + 1 <= last);
      tile_pair<1, WFIRST>(tb, st, scr, as, bs, raw, sraw, pk, acc, cw0, last, q + 1, lane, r32, h, c + 2 <= last,
                           c + 3 <= last);
    }
  }
}

// ---- weights in operand order -------------------------------------------------------
//
// The packed copy of the experts (moe_prefill_pack_weights) holds each matrix
// as blocks of 32 rows x one chunk pair: four K-steps of 64 lanes x 16 code
// bytes (lane l: row l % 32, bytes 16 (l / 32) of the K-step's 32), then 64
// lanes x 4 scale bytes (byte S: the scale of block 2 S + l / 32 of the pair).
// A wavefront then loads each fragment's K-step operand as one contiguous
// 1 KB straight into the register the MFMA reads and its scale word in one
// 256-byte load: no trip through LDS, no reordering, and two lines of scales
// per fragment and pair instead of 32.  The small-bucket kernels read the
// same blocks (a unit's 32 gate and 32 up rows, or 64 down rows, are whole
// row blocks).

constexpr int kPkBlock = 4096 + 256;  // bytes of a (32-row block, chunk pair) of the packed copy

__host__ __device__ inline int pk_pairs(int K) { return (K + 255) / 256; }
// Bytes of one slot of the packed copy: gate, up (I rows of H), then down (H rows of I).
__host__ __device__ inline size_t pk_slot_bytes(int H, int I) {
  return ((size_t)2 * (I / 32) * pk_pairs(H) + (size_t)(H / 32) * pk_pairs(I)) * kPkBlock;
}

struct BSrcPk {
  rsrc_t r;        // the slot's packed blocks
  uint32_t fb[2];  // the lane's code bytes in fragment g's first block, kOob past the matrix
  uint32_t sb[2];  // the lane's scale word in that block
  __device__ __forceinline__ void init(rsrc_t rr, uint32_t base0, uint32_t base1, bool live0, bool live1, int lane) {
    r = rr;
    fb[0] = live0 ? base0 + 16u * (uint32_t)lane : kOob;
    fb[1] = live1 ? base1 + 16u * (uint32_t)lane : kOob;
    sb[0] = live0 ? base0 + 4096u + 4u * (uint32_t)lane : kOob;
    sb[1] = live1 ? base1 + 4096u + 4u * (uint32_t)lane : kOob;
  }
  // Fragment g's operand of K-step S of pair pq; pq < 0 loads zeros.
  __device__ __forceinline__ uint4_t step(int g, int pq, int S) const {
    return bload16(r, pq < 0 || fb[g] == kOob ? kOob : fb[g] + (uint32_t)pq * kPkBlock + (uint32_t)S * 1024u);
  }
  // Fragment g's scale word of pair pq (byte S: K-step S).
  __device__ __forceinline__ uint32_t scales(int g, int pq) const {
    return bload4(r, pq < 0 || sb[g] == kOob ? kOob : sb[g] + (uint32_t)pq * kPkBlock);
  }
};

// Pair q of a window with operand-order weights.  Loads: the activation
// copies of the next pair go out first; then each K-step's registers are
// reloaded with the next pair's operand as soon as its MFMAs are issued, and
// the next pair's scale words go out with the first of them, so each K-step
// waits only for its own operands.  One barrier per pair, for the activation
// stages.
template <int PJ, bool WFIRST>
__device__ __forceinline__ void tile_pair_pk(const TileTables& tb, uint8_t* const (&st)[4], const ACopy& as,
                                             const BSrcPk& bs, uint4_t (&bq)[2][4], uint32_t (&ws)[2],
                                             f16v (&acc)[4][2], int cw0, int last, int q, int r32, int h, bool run0,
                                             bool run1) {
  const int c0 = cw0 + 2 * q, n0 = c0 + 2;
  const int pqn = n0 <= last ? n0 / 2 : -1;
  as.copy(st[2 - 2 * PJ], n0 <= last ? n0 : -1);
  as.copy(st[3 - 2 * PJ], n0 + 1 <= last ? n0 + 1 : -1);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t wsn[2];
#pragma unroll
  for (int S = 0; S < 4; ++S) {
    if (S < 2 ? run0 : run1) {
      const uint8_t* sta = st[2 * PJ + (S >> 1)];
      const uint4_t sa = scale_words(tb.sca, c0 + (S >> 1) - cw0, r32, h);
      i8v a[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) a[f] = (S & 1) ? read_afrag<1>(sta, f, r32, h) : read_afrag<0>(sta, f, r32, h);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int sw = (int)ws[g];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (S == 0) acc[f][g] = tile_mfma<WFIRST, 0, 0>(bop(bq[g][S]), a[f], acc[f][g], sw, word(sa, f));
          if (S == 1) acc[f][g] = tile_mfma<WFIRST, 1, 2>(bop(bq[g][S]), a[f], acc[f][g], sw, word(sa, f));
          if (S == 2) acc[f][g] = tile_mfma<WFIRST, 2, 0>(bop(bq[g][S]), a[f], acc[f][g], sw, word(sa, f));
          if (S == 3) acc[f][g] = tile_mfma<WFIRST, 3, 2>(bop(bq[g][S]), a[f], acc[f][g], sw, word(sa, f));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (S == 0) {
#pragma unroll
      for (int g = 0; g < 2; ++g) wsn[g] = bs.scales(g, pqn);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) bq[g][S] = bs.step(g, pqn, S);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) ws[g] = wsn[g];
  wait_vm<kPairPkVm>();  // this wavefront's copies of the next pair are done
  wg_barrier();
}

// All K of one tile with operand-order weights (see tile_k_loop).  The first
// pair's scale words are loaded before its operands, as in every later pair,
// so that each K-step's wait counts the same loads.
template <bool WFIRST, typename Tables>
__device__ __forceinline__ void tile_k_loop_pk(TileTables& tb, uint8_t* const (&st)[4], f16v (&acc)[4][2],
                                               const ACopy& as, const BSrcPk& bs, int nch, int tid, Tables tables) {
  const int lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  for (int cw0 = 0; cw0 < nch; cw0 += TWIN) {
    const int last = min(cw0 + TWIN, nch) - 1;
    if (cw0 > 0) wg_barrier();  // every wavefront is done with the previous window
    as.copy(st[0], cw0);
    as.copy(st[1], cw0 + 1 <= last ? cw0 + 1 : -1);
    tables(cw0);
    __builtin_amdgcn_sched_barrier(0);
    uint4_t bq[2][4];
    uint32_t ws[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) ws[g] = bs.scales(g, cw0 / 2);
#pragma unroll
    for (int S = 0; S < 4; ++S)
#pragma unroll
      for (int g = 0; g < 2; ++g) bq[g][S] = bs.step(g, cw0 / 2, S);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kPairPkVm>();  // all but the weight loads just issued
    wait_lgkm0();          // the table stores
    wg_barrier();
    for (int q = 0; cw0 + 2 * q <= last; q += 2) {
      const int c = cw0 + 2 * q;
      tile_pair_pk<0, WFIRST>(tb, st, as, bs, bq, ws, acc, cw0, last, q, r32, h, true, c + 1 <= last);
      tile_pair_pk<1, WFIRST>(tb, st, as, bs, bq, ws, acc, cw0, last, q + 1, r32, h, c + 2 <= last, c + 3 <= last);
    }
  }
}

// SwiGLU of the GEMM epilogues: silu(g) = g / (1 + 2^(-g log2 e)) on the
// hardware exp2 and reciprocal (about one ulp each; h then goes to MXFP6, whose
// step is 2^-3 of the block's scale).  Saturates to 0 for g below about -88 and
// to g * u above about +17, like the exact form.
__device__ __forceinline__ float swiglu_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---- streaming path for small buckets ----------------------------------------------
//
// A bucket of at most SK_MAX rows (most experts of a prefill chunk: tokens
// spread thinly over the routed experts) is a weight stream, not a GEMM: its
// expert is read once for a handful of rows.  One wavefront per (bucket, 32
// weight rows of each of two matrices): its A fragment (the bucket's rows,
// rows past the end read as zeros) comes from memory into registers in MFMA
// order and its two B fragments in 8-row loads, in batches of four K-steps,
// and many wavefronts per CU keep the HBM stream full.


// Four K-steps (two 128-K chunks) of one wavefront: A, the lane's 48-byte
// record (row r32, K-half h) of each chunk in three 16-byte loads (K-step 2c
// takes its bytes 0-23, block 2c... of the record, K-step 2c+1 bytes 24-47);
// each B fragment's 32 rows x 128 B of the two chunks as loaded, four loads of
// 8 rows (b[g][j]: rows 8 j + l / 8, bytes 16 (l % 8)), moved into MFMA order
// through the wavefront's LDS area when used (a load over the 16 or 32 rows of
// an operand streams at about two thirds of this rate from memory).
struct SkRegs {
  uint4_t a[2][3];  // [chunk][16 B of the lane's 48-byte record]: K-step 2c bytes 0-23, 2c+1 bytes 24-47
  uint4_t b[2][4];  // [fragment][load] (packed weights: [fragment][K-step], in operand order)
  uint32_t ws[2];   // packed weights: each fragment's scale word of the pair (byte S: K-step S)
};

// Scale words come from a per-wavefront LDS table read once per window of
// SKWIN chunks: rows 0-31 the unit's A rows, 32-63 and 64-95 its two weight
// fragments (whose scale bytes are contiguous).
constexpr int SKWIN = 20;
constexpr int SKW = SKWIN + 1;  // words per table row (odd: 32 rows hit 32 banks)
constexpr int SK_SCR = 32 * 128;  // a wavefront's LDS area for one fragment's two chunks in MFMA order

struct SkSrc {
  rsrc_t ra, rb[2];
  uint32_t va, vb[2];  // va: the lane's record (row r32, K-half h) in chunk 0; vb: row l / 8 of the fragment, + 16 (l % 8)
  uint32_t cstride;    // bytes per chunk of the A records
  uint32_t row8;       // bytes from a weight row to the row 8 below
  rsrc_t rp;           // packed weights: the slot's blocks
  uint32_t pb[2];      // packed weights: the lane's code bytes in fragment g's first block
  template <bool PK>
  __device__ __forceinline__ void load(int n, SkRegs& r) const {
#pragma unroll
    for (int c = 0; c < 2; ++c) {  // chunk 2n + c: the lane's whole record (records are 48 B, 16-B aligned)
      const uint32_t o = va + (uint32_t)(2 * n + c) * cstride;
#pragma unroll
      for (int j = 0; j < 3; ++j) r.a[c][j] = bload16(ra, o + 16u * j);
    }
    if constexpr (PK) {
      // the pair's scale words first, then its four K-step operands per fragment
#pragma unroll
      for (int g = 0; g < 2; ++g)
        r.ws[g] = bload4(rp, pb[g] + (uint32_t)n * kPkBlock + 4096u - 12u * (uint32_t)(__lane_id()));
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int S = 0; S < 4; ++S) r.b[g][S] = bload16(rp, pb[g] + (uint32_t)n * kPkBlock + (uint32_t)S * 1024u);
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) r.b[g][j] = bload16(rb[g], vb[g] + (uint32_t)j * row8 + (uint32_t)n * 128u);
    }
  }
};

// A fragment's four K-step operands from its loads (b: as SkRegs::b[g]): the
// rows are written into the wavefront's LDS area in operand order (K-step S at
// S * 1024, lane t's 16 B at slot t ^ 2 S, so both the writes and the reads
// stay within two LDS banks per slot) and read back.  A wavefront's LDS
// accesses complete in order, so the area serves one fragment after another.
__device__ __forceinline__ void sk_operands(const uint4_t (&b)[4], uint8_t* scr, i8v (&op)[4]) {
  const int lane = __lane_id(), r8 = lane >> 3, s = lane & 7, S = s >> 1, hh = s & 1;
  uint8_t* wr = scr + S * 1024 + ((r8 ^ (2 * S)) + 32 * hh) * 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4_t*>(wr + j * 128) = b[j];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint4_t q = *reinterpret_cast<const uint4_t*>(scr + k * 1024 + ((lane ^ (2 * k)) * 16));
    op[k] = i8v{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  }
}

template <bool PK>
__device__ __forceinline__ void sk_mma(const SkRegs& r, f16v (&acc)[2], int nks, int h, const uint32_t* tab,
                                       int cw, uint8_t* scr) {  // cw: the batch's first chunk within the window
  const int r32 = __lane_id() & 31;
  i8v bop[2][4];  // [fragment][K-step]
  if constexpr (PK) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int k = 0; k < 4; ++k) bop[g][k] = i8v{(int)r.b[g][k].x, (int)r.b[g][k].y, (int)r.b[g][k].z, (int)r.b[g][k].w, 0, 0, 0, 0};
  } else {
#pragma unroll
    for (int g = 0; g < 2; ++g) sk_operands(r.b[g], scr, bop[g]);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < nks) {
      // K-step s: block 2(s%2) + h = bytes 24 (s%2) .. of the record of chunk 2n + s/2
      const uint4_t* q = r.a[s >> 1];
      const i8v a = (s & 1) ? i8v{(int)q[1].z, (int)q[1].w, (int)q[2].x, (int)q[2].y, (int)q[2].z, (int)q[2].w, 0, 0}
                            : i8v{(int)q[0].x, (int)q[0].y, (int)q[0].z, (int)q[0].w, (int)q[1].x, (int)q[1].y, 0, 0};
      // low byte: the scale of block 2s+h
      const int sa = (int)((tab[r32 * SKW + cw + (s >> 1)] >> (8 * h)) >> (16 * (s & 1)));
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if constexpr (PK) {
          const int sb = (int)r.ws[g];  // byte s: K-step s
          if (s == 0) acc[g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[g][s], acc[g], 2, 4, 0, sa, 0, sb);
          if (s == 1) acc[g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[g][s], acc[g], 2, 4, 0, sa, 1, sb);
          if (s == 2) acc[g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[g][s], acc[g], 2, 4, 0, sa, 2, sb);
          if (s == 3) acc[g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[g][s], acc[g], 2, 4, 0, sa, 3, sb);
        } else {
          const int sb = (int)((tab[(32 + 32 * g + r32) * SKW + cw + (s >> 1)] >> (8 * h)) >> (16 * (s & 1)));
          acc[g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[g][s], acc[g], 2, 4, 0, sa, 0, sb);
        }
      }
    }
  }
}

// The scale tables of a unit's window: its A rows (loader AS) and its two
// weight fragments.
template <typename AS>
struct SkTables {
  AS a;
  ScaleRows<32, 64, SKWIN, SKW> b[2];
};

// All K of one unit: batches of four K-steps, each batch's loads issued once
// the previous batch's MFMAs have read their registers.  One batch in flight
// per wavefront streams faster than two once the rows live beyond L2 (fewer
// loads queued per wavefront), and the eight wavefronts of a CU cover each
// other's waits.  The load after the last batch re-reads it (never used): no
// load behind a branch.  tables(cw0, ts) issues the scale-table loads of the
// window starting at chunk cw0.
template <typename TS, bool PK, typename Tables>
__device__ __forceinline__ void sk_k_loop(const SkSrc& src, f16v (&acc)[2], int K, int h, uint32_t* tab,
                                          uint8_t* scr, Tables tables) {
  const int nks_total = K / 64, nchunks = K / KC;
  const int lane = __lane_id();
  for (int cw0 = 0; cw0 < nchunks; cw0 += SKWIN) {
    const int b0 = cw0 / 2, last = (min(cw0 + SKWIN, nchunks) + 1) / 2 - 1;  // batches of this window
    TS ts;
    tables(cw0, ts);
    SkRegs r0;
    src.load<PK>(b0, r0);
    ts.a.store(tab, lane);
    if constexpr (!PK) {
      ts.b[0].store(tab + 32 * SKW, lane);
      ts.b[1].store(tab + 64 * SKW, lane);
    }
    __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses complete in order
    for (int n = b0; n <= last; ++n) {
      sk_mma<PK>(r0, acc, min(4, nks_total - 4 * n), h, tab, 2 * (n - b0), scr);
      src.load<PK>(min(n + 1, last), r0);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The streaming kernels launch one wavefront per possible unit (four per
// workgroup); those past the plan's unit count exit at once, and the hardware
// dispatcher balances the rest.

template <bool PK>  // PK: weights from the packed copy pk (operand order), else the row-major store
__global__ __launch_bounds__(kPT, 2) void gateup_skinny_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, uint32_t xq_bytes, uint32_t xs_bytes, int P,
    ExpertStore w, const uint8_t* __restrict__ pk, const int32_t* __restrict__ sorted_pair, const SkBucket* __restrict__ sbk,
    const int32_t* __restrict__ counts, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ float stage[4][32 * 33];
  __shared__ uint32_t sktab[4][96 * SKW];
  __shared__ __attribute__((aligned(16))) uint8_t skscr[4][SK_SCR];
  const int H = w.H, I = w.I, NBH = H / 32, NBI = I / 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, r32 = lane & 31, h = lane >> 5;
  const uint32_t wrow = (uint32_t)H / 2u;
  const size_t mat = (size_t)I * wrow, smat = (size_t)I * NBH;
  const int groups = I / 32, units = counts[2] * groups;
  float* st = stage[wid];
  for (int u = blockIdx.x * 4 + wid; u < units; u += gridDim.x * 4) {
    const SkBucket bk = sbk[u / groups];
    const int q = u % groups;
    if (bk.slot < 0) continue;
    SkSrc src;
    src.ra = make_rsrc(xq, xq_bytes);
    src.va = r32 < bk.cnt ? ((uint32_t)h * (uint32_t)P + (uint32_t)(bk.row0 + r32)) * 48u : kOob;
    src.cstride = 96u * (uint32_t)P;
    src.rb[0] = make_rsrc(w.wg + (size_t)bk.slot * mat, (uint32_t)mat);
    src.rb[1] = make_rsrc(w.wu + (size_t)bk.slot * mat, (uint32_t)mat);
    src.vb[0] = src.vb[1] = (uint32_t)(32 * q + (lane >> 3)) * wrow + 16u * (uint32_t)(lane & 7);
    src.row8 = 8u * wrow;
    if constexpr (PK) {
      const size_t sbytes = pk_slot_bytes(H, I);
      const uint32_t np = (uint32_t)pk_pairs(H);
      src.rp = make_rsrc(pk + (size_t)bk.slot * sbytes, (uint32_t)sbytes);
      src.pb[0] = (uint32_t)q * np * (uint32_t)kPkBlock + 16u * (uint32_t)lane;
      src.pb[1] = src.pb[0] + (uint32_t)(I / 32) * np * (uint32_t)kPkBlock;  // the up matrix
    }
    const rsrc_t xsr = make_rsrc(xs, xs_bytes);
    const rsrc_t sgr = make_rsrc(w.sg + (size_t)bk.slot * smat, (uint32_t)smat);
    const rsrc_t sur = make_rsrc(w.su + (size_t)bk.slot * smat, (uint32_t)smat);
    using TS = SkTables<ScaleCols<32, 64, SKWIN, SKW>>;
    auto tables = [&](int cw0, TS& ts) {
      ts.a.issue(xsr, cw0, lane, bk.row0, bk.cnt, P);
      if constexpr (!PK) {
        ts.b[0].issue(sgr, cw0, lane, [&](int r) { return (uint32_t)(32 * q + r) * NBH; });
        ts.b[1].issue(sur, cw0, lane, [&](int r) { return (uint32_t)(32 * q + r) * NBH; });
      }
    };
    f16v acc[2] = {f16v{}, f16v{}};
    sk_k_loop<TS, PK>(src, acc, H, h, sktab[wid], skscr[wid], tables);
    // h = silu(g) * u: rows of the bucket x this unit's 32 h columns (one MXFP6 block per row)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + h * 4 + (i & 3);
      st[row * 33 + r32] = swiglu_fast(acc[0][i], acc[1][i]);
    }
    __builtin_amdgcn_wave_barrier();
    if (h == 0 && r32 < bk.cnt) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = st[r32 * 33 + i];
      uint32_t pk[6], sb;
      q6_block(v, pk, sb);
      const size_t grow = (size_t)(bk.row0 + r32);
      uint2* dst = reinterpret_cast<uint2*>(hq + q6_offset(bk.row0 + r32, q, P));
      dst[0] = make_uint2(pk[0], pk[1]);
      dst[1] = make_uint2(pk[2], pk[3]);
      dst[2] = make_uint2(pk[4], pk[5]);
      hs[grow * NBI + q] = (uint8_t)sb;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <bool PK>
__global__ __launch_bounds__(kPT, 2) void down_skinny_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, uint32_t hq_bytes, uint32_t hs_bytes, int P,
    ExpertStore w, const uint8_t* __restrict__ pk, const int32_t* __restrict__ sorted_pair, const SkBucket* __restrict__ sbk,
    const int32_t* __restrict__ counts, float* __restrict__ y) {
  __shared__ uint32_t sktab[4][96 * SKW];
  __shared__ __attribute__((aligned(16))) uint8_t skscr[4][SK_SCR];
  const int H = w.H, I = w.I, NBI = I / 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, r32 = lane & 31, h = lane >> 5;
  const uint32_t wrow = (uint32_t)I / 2u;
  const size_t mat = (size_t)H * wrow, smat = (size_t)H * NBI;
  const int groups = H / 64, units = counts[2] * groups;
  for (int u = blockIdx.x * 4 + wid; u < units; u += gridDim.x * 4) {
    const SkBucket bk = sbk[u / groups];
    const int n0 = 64 * (u % groups);
    if (bk.slot < 0) {
      // no stored expert: its rows are zero
      for (int r = 0; r < bk.cnt; ++r) y[(size_t)sorted_pair[bk.row0 + r] * H + n0 + lane] = 0.f;
      continue;
    }
    SkSrc src;
    src.ra = make_rsrc(hq, hq_bytes);
    src.va = r32 < bk.cnt ? ((uint32_t)h * (uint32_t)P + (uint32_t)(bk.row0 + r32)) * 48u : kOob;
    src.cstride = 96u * (uint32_t)P;
    const rsrc_t rc = make_rsrc(w.wd + (size_t)bk.slot * mat, (uint32_t)mat);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      src.rb[g] = rc;
      src.vb[g] = (uint32_t)(n0 + 32 * g + (lane >> 3)) * wrow + 16u * (uint32_t)(lane & 7);
    }
    src.row8 = 8u * wrow;
    if constexpr (PK) {
      const size_t sbytes = pk_slot_bytes(H, I);
      const uint32_t np = (uint32_t)pk_pairs(I), rb = (uint32_t)n0 / 32u;
      const uint32_t dn0 = 2u * (uint32_t)(I / 32) * (uint32_t)pk_pairs(H) * (uint32_t)kPkBlock;  // first down block
      src.rp = make_rsrc(pk + (size_t)bk.slot * sbytes, (uint32_t)sbytes);
      src.pb[0] = dn0 + rb * np * (uint32_t)kPkBlock + 16u * (uint32_t)lane;
      src.pb[1] = src.pb[0] + np * (uint32_t)kPkBlock;
    }
    const rsrc_t hsr = make_rsrc(hs, hs_bytes);
    const rsrc_t sdr = make_rsrc(w.sd + (size_t)bk.slot * smat, (uint32_t)smat);
    using TS = SkTables<ScaleRows<32, 64, SKWIN, SKW>>;
    auto tables = [&](int cw0, TS& ts) {
      ts.a.issue(hsr, cw0, lane, [&](int r) { return r < bk.cnt ? (uint32_t)(bk.row0 + r) * NBI : kOob; });
      if constexpr (!PK) {
        ts.b[0].issue(sdr, cw0, lane, [&](int r) { return (uint32_t)(n0 + r) * NBI; });
        ts.b[1].issue(sdr, cw0, lane, [&](int r) { return (uint32_t)(n0 + 32 + r) * NBI; });
      }
    };
    f16v acc[2] = {f16v{}, f16v{}};
    sk_k_loop<TS, PK>(src, acc, I, h, sktab[wid], skscr[wid], tables);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + h * 4 + (i & 3);
      if (row < bk.cnt) {
        float* yr = y + (size_t)sorted_pair[bk.row0 + row] * H + n0 + r32;
        __builtin_nontemporal_store(acc[0][i], yr);  // streaming stores, as in the tiled down GEMM
        __builtin_nontemporal_store(acc[1][i], yr + 32);
      }
    }
  }
}

// ---- P1: gate/up GEMM, SwiGLU and MXFP6 of h -----------------------------------------
//
// Wavefront w of a tile owns h columns j0 + 64 w .. j0 + 64 w + 63: its four
// fragments are those gate rows (two) and the same up rows (two), so
// h = silu(g) * u is formed in its registers.  The tile's 256 h columns are
// staged in LDS and quantised per (row, 32-column block) into hq/hs.  In a
// last tile narrower than 256 columns (inter % 256 == 128) wavefronts 2 and 3
// load zeros and store nothing.

template <bool PK>  // PK: weights from the packed copy pk (operand order), else the row-major store
__global__ __launch_bounds__(kTilePT, 1) void gateup_tile_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, uint32_t xq_bytes, uint32_t xs_bytes, int P,
    ExpertStore w, const uint8_t* __restrict__ pk, const TileDesc* __restrict__ tiles,
    const int32_t* __restrict__ counts, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ TileTables tb;
  __shared__ __attribute__((aligned(16))) uint8_t a0[A_STAGE], a1[A_STAGE], a2[A_STAGE], a3[A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t bscr[PK ? 16 : 8 * B_SCR];
  uint8_t* const st[4] = {a0, a1, a2, a3};
  const int H = w.H, I = w.I, NBH = H / 32, NBI = I / 32;
  // wid in a scalar register: every address derived from it alone stays scalar
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6), r32 = lane & 31;
  const uint32_t wrow = (uint32_t)H / 2u;
  const size_t mat = (size_t)I * wrow, smat = (size_t)I * NBH;
  const int total = counts[0];
  // Every K loop ends on a barrier after the last reads of the stages and the
  // table, and the epilogue uses registers only, so a tile can start at once.
  for (TileWalk tw(total); tw.next < tw.end; tw.next += tw.step) {
    const TileDesc d = tiles[tw.next];
    if (d.slot < 0) continue;  // no stored expert: the down GEMM writes its rows as zeros
    const int j0 = d.ntile * GU_N;
    const int hc0 = j0 + 32 * wid;  // this wavefront's 32 h columns: gate rows hc0.. (fragment 0), up rows (1)
    const bool live = hc0 < I;      // inter % 256 == 128: the last tile is half wide
    ACopy as;
    as.init(xq, xq_bytes, wid, lane, d.row0, P);
    BSrc bs;
    BSrcPk bp;
    if constexpr (PK) {
      const size_t sbytes = pk_slot_bytes(H, I);
      const uint32_t np = (uint32_t)pk_pairs(H), rb = (uint32_t)hc0 / 32u;
      const uint32_t up0 = (uint32_t)(I / 32) * np * (uint32_t)kPkBlock;  // the up matrix's first block
      bp.init(make_rsrc(pk + (size_t)d.slot * sbytes, (uint32_t)sbytes), rb * np * (uint32_t)kPkBlock,
              up0 + rb * np * (uint32_t)kPkBlock, live, live, lane);
    } else {
      bs.rc[0] = make_rsrc(w.wg + (size_t)d.slot * mat, (uint32_t)mat);
      bs.rc[1] = make_rsrc(w.wu + (size_t)d.slot * mat, (uint32_t)mat);
      bs.rs[0] = make_rsrc(w.sg + (size_t)d.slot * smat, (uint32_t)smat);
      bs.rs[1] = make_rsrc(w.su + (size_t)d.slot * smat, (uint32_t)smat);
      bs.row8 = 8u * wrow;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        bs.vc[g] = live ? ((uint32_t)hc0 + (uint32_t)(lane >> 3)) * wrow + 16u * (uint32_t)(lane & 7) : kOob;
        bs.vs[g] = live ? ((uint32_t)hc0 + (uint32_t)r32) * (uint32_t)NBH + 8u * (uint32_t)(lane >> 5) : kOob;
      }
    }
    const rsrc_t xsr = make_rsrc(xs, xs_bytes);
    auto tables = [&](int cw0) {
      const int t = opaque(tid);
      ScaleCols<BM, kTilePT, TWIN, TWIN + 1> ta;
      ta.issue(xsr, cw0, t, d.row0, d.mrows, P);
      ta.store_cf(tb.sca, t);
    };
    f16v acc[4][2];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f][0] = acc[f][1] = f16v{};
    if constexpr (PK) tile_k_loop_pk<true>(tb, st, acc, as, bp, H / KC, tid, tables);  // ends on a barrier
    else tile_k_loop<true>(tb, st, bscr + wid * B_SCR, acc, as, bs, H / KC, tid, tables);
    // h = silu(g) * u and its MXFP6 block, in registers.  Lane l holds row
    // 32 f + l % 32 and columns 8 j + 4 (l / 32) + i of the wavefront's 32 in
    // register 4 j + i: the block's largest magnitude and its packed codes are
    // completed with the partner lane l ^ 32.
    if (live) {
      const int t = opaque(tid), e32 = t & 31, eh = (t >> 5) & 1;
      const int gblk = hc0 >> 5;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int row = 32 * f + e32;
        float hv[16], amax = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          hv[r] = swiglu_fast(acc[f][0][r], acc[f][1][r]);
          amax = fmaxf(amax, fabsf(hv[r]));
        }
        const auto mx = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(mx[0]), __uint_as_float(mx[1]));
        // G[j]: the four codes of columns 8 j + 4 eh .. + 3 (24 bits)
        uint32_t G[4] = {0u, 0u, 0u, 0u}, sbyte = 0u;
        if (amax != 0.f) {
          float inv;
          sbyte = q6_scale(amax, inv);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) G[j] |= e2m3_rne(hv[4 * j + i] * inv) << (6 * i);
        }
        // The record's 24 bytes: code m at bits 6m..6m+5, so columns 8j'..8j'+7
        // are 48 bits, the lower lane's G[j'] then the upper lane's.  The lower
        // lane writes bytes 0-11 (j' = 0, 1), the upper lane bytes 12-23.
        const uint32_t s0 = eh ? G[0] : G[2], s1 = eh ? G[1] : G[3];
        const auto x0 = __builtin_amdgcn_permlane32_swap(s0, s0, false, false);
        const auto x1 = __builtin_amdgcn_permlane32_swap(s1, s1, false, false);
        const uint32_t q0 = eh ? x0[0] : x0[1], q1 = eh ? x1[0] : x1[1];
        const uint32_t lo0 = eh ? q0 : G[0], lo1 = eh ? q1 : G[1], hi0 = eh ? G[2] : q0, hi1 = eh ? G[3] : q1;
        if (row < d.mrows) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(hq + q6_offset(d.row0 + row, gblk, P) + 12 * eh);
          dst[0] = lo0 | (hi0 << 24);
          dst[1] = (hi0 >> 8) | (lo1 << 16);
          dst[2] = (lo1 >> 16) | (hi1 << 8);
          if (eh == 0) hs[(size_t)(d.row0 + row) * NBI + gblk] = (uint8_t)sbyte;
        }
      }
    }
  }
  wait_vm<0>();  // no copy into LDS outlives the workgroup
}

// ---- P2: down GEMM -> y_pair ---------------------------------------------------------
//
// Wavefront w of a tile owns output columns n0 + 64 w .. + 63 (two fragments
// of W_down rows); each lane stores its accumulators straight into the y_pair
// rows of the tile's pairs (32 consecutive columns of two rows per store).  In
// a last tile narrower than 512 columns (hidden % 512 == 256) wavefronts 4-7
// load zeros and store nothing.

template <bool PK>
__global__ __launch_bounds__(kTilePT, 1) void down_tile_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, uint32_t hq_bytes, uint32_t hs_bytes, int P,
    ExpertStore w, const uint8_t* __restrict__ pk, const int32_t* __restrict__ sorted_pair,
    const TileDesc* __restrict__ tiles, const int32_t* __restrict__ counts, float* __restrict__ y) {
  __shared__ TileTables tb;
  __shared__ __attribute__((aligned(16))) uint8_t a0[A_STAGE], a1[A_STAGE], a2[A_STAGE], a3[A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t bscr[PK ? 16 : 8 * B_SCR];
  __shared__ int rowtok[BM];
  uint8_t* const st[4] = {a0, a1, a2, a3};
  const int H = w.H, I = w.I, NBI = I / 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6), r32 = lane & 31;
  const uint32_t wrow = (uint32_t)I / 2u;
  const size_t mat = (size_t)H * wrow, smat = (size_t)H * NBI;
  const int total = counts[1];
  for (TileWalk tw(total); tw.next < tw.end; tw.next += tw.step) {
    const TileDesc d = tiles[tw.next];
    wg_barrier();  // the previous tile's epilogue has read rowtok
    if (tid < BM) rowtok[tid] = tid < d.mrows ? sorted_pair[d.row0 + tid] : -1;
    wait_lgkm0();
    wg_barrier();
    const int n0 = d.ntile * DN_N;
    const int nc0 = n0 + WN * wid;  // this wavefront's first output column
    const bool live = nc0 < H;
    if (d.slot < 0) {
      for (int i = tid; i < d.mrows * DN_N; i += kTilePT) {
        const int row = i / DN_N, col = i % DN_N;
        if (n0 + col < H) y[(size_t)rowtok[row] * H + n0 + col] = 0.f;
      }
      continue;
    }
    ACopy as;
    as.init(hq, hq_bytes, wid, lane, d.row0, P);
    BSrc bs;
    BSrcPk bp;
    if constexpr (PK) {
      const size_t sbytes = pk_slot_bytes(H, I);
      const uint32_t np = (uint32_t)pk_pairs(I), rb = (uint32_t)nc0 / 32u;
      const uint32_t dn0 = 2u * (uint32_t)(I / 32) * (uint32_t)pk_pairs(H) * (uint32_t)kPkBlock;  // first down block
      bp.init(make_rsrc(pk + (size_t)d.slot * sbytes, (uint32_t)sbytes), dn0 + rb * np * (uint32_t)kPkBlock,
              dn0 + (rb + 1u) * np * (uint32_t)kPkBlock, live, live, lane);
    } else {
      const rsrc_t rd = make_rsrc(w.wd + (size_t)d.slot * mat, (uint32_t)mat);
      const rsrc_t sdr = make_rsrc(w.sd + (size_t)d.slot * smat, (uint32_t)smat);
      bs.row8 = 8u * wrow;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t row = (uint32_t)(nc0 + 32 * g);
        bs.rc[g] = rd;
        bs.rs[g] = sdr;
        bs.vc[g] = live ? (row + (uint32_t)(lane >> 3)) * wrow + 16u * (uint32_t)(lane & 7) : kOob;
        bs.vs[g] = live ? (row + (uint32_t)r32) * (uint32_t)NBI + 8u * (uint32_t)(lane >> 5) : kOob;
      }
    }
    const rsrc_t hsr = make_rsrc(hs, hs_bytes);
    auto tables = [&](int cw0) {
      // hs is row-major [sorted row][I/32], so its words are read row by row
      const int t = opaque(tid);
      ScaleRows<BM, kTilePT, TWIN, TWIN + 1> ta;
      ta.issue(hsr, cw0, t, [&](int r) { return r < d.mrows ? (uint32_t)(d.row0 + r) * (uint32_t)NBI : kOob; });
      ta.store_cf(tb.sca, t);
    };
    f16v acc[4][2];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f][0] = acc[f][1] = f16v{};
    if constexpr (PK) tile_k_loop_pk<false>(tb, st, acc, as, bp, I / KC, tid, tables);
    else tile_k_loop<false>(tb, st, bscr + wid * B_SCR, acc, as, bs, I / KC, tid, tables);
    if (live) {
      const int t = opaque(tid), e32 = t & 31, eh = (t >> 5) & 1;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        __builtin_amdgcn_sched_barrier(0);  // one fragment's stores at a time (register pressure)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * f + (r >> 2) * 8 + eh * 4 + (r & 3);
          if (row < d.mrows) {
            float* yr = y + (size_t)rowtok[row] * H + nc0 + e32;
            // streaming stores: the rows are read once, by the combine, after the whole
            // GEMM (671 MB at 4096 tokens), so caching them only leaves dirty lines to evict
#pragma unroll
            for (int g = 0; g < 2; ++g) __builtin_nontemporal_store(acc[f][g][r], yr + 32 * g);
          }
        }
      }
    }
  }
  wait_vm<0>();  // no copy into LDS outlives the workgroup
}

// ---- the packed copy ------------------------------------------------------------------
//
// One thread per (slot, matrix, 32-row block, chunk pair, lane): it gathers
// the lane's 16 code bytes of each K-step and its four scale bytes from the
// row-major store (zeros past K) and writes them where the operand-order
// loads read them, 1 KB per K-step and wavefront.
__global__ __launch_bounds__(256) void pack_weights_kernel(ExpertStore w, uint8_t* __restrict__ dst) {
  const int H = w.H, I = w.I, slot = blockIdx.y;
  const long u = (long)blockIdx.x * 256 + threadIdx.x;
  const int npg = pk_pairs(H), npd = pk_pairs(I);
  const long ngu = (long)(I / 32) * npg, ndn = (long)(H / 32) * npd;
  const long blk = u >> 6;
  if (blk >= 2 * ngu + ndn) return;
  const int t = (int)(u & 63), r32 = t & 31, h = t >> 5;
  int K, np;
  long b;
  const uint8_t *codes, *scales;
  if (blk < 2 * ngu) {
    const int m = blk < ngu ? 0 : 1;
    b = blk - m * ngu;
    K = H;
    np = npg;
    codes = (m ? w.wu : w.wg) + (size_t)slot * I * (H / 2);
    scales = (m ? w.su : w.sg) + (size_t)slot * I * (H / 32);
  } else {
    b = blk - 2 * ngu;
    K = I;
    np = npd;
    codes = w.wd + (size_t)slot * H * (I / 2);
    scales = w.sd + (size_t)slot * H * (I / 32);
  }
  const long rb = b / np;
  const int pq = (int)(b - rb * np);
  const long row = rb * 32 + r32;
  const int KB = K / 2, NB = K / 32;
  uint8_t* o = dst + (size_t)slot * pk_slot_bytes(H, I) + (size_t)blk * kPkBlock;
#pragma unroll
  for (int S = 0; S < 4; ++S) {
    const int off = 128 * pq + 32 * S + 16 * h;  // the lane's code bytes of K-step S within the row
    uint4_t v = {0u, 0u, 0u, 0u};
    if (off < KB) v = *reinterpret_cast<const uint4_t*>(codes + (size_t)row * KB + off);
    *reinterpret_cast<uint4_t*>(o + S * 1024 + 16 * t) = v;
  }
  uint32_t word = 0u;
#pragma unroll
  for (int S = 0; S < 4; ++S) {
    const int blkk = 8 * pq + 2 * S + h;  // scale block of K-step S for this lane
    if (blkk < NB) word |= (uint32_t)scales[(size_t)row * NB + blkk] << (8 * S);
  }
  *reinterpret_cast<uint32_t*>(o + 4096 + 4 * t) = word;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Upper bound of the row tiles of a call: one ragged tile per non-empty bucket.
size_t max_mtiles(size_t P) { return (P + BM - 1) / BM + (P < (size_t)kMaxExperts ? P : (size_t)kMaxExperts); }

}  // namespace

size_t prefill_workspace_bytes(int T, int k, int H, int I) {
  const size_t P = (size_t)T * k, nm = max_mtiles(P);
  return align256(P * H / 32 * 24) + align256(P * H / 32) + align256(P * I / 32 * 24) +
         align256(P * I / 32) + align256(nm * ((I + GU_N - 1) / GU_N) * sizeof(TileDesc)) +
         align256(nm * ((H + DN_N - 1) / DN_N) * sizeof(TileDesc)) + align256(kMaxExperts * sizeof(SkBucket)) + 256 +
         align256((size_t)T * H / 32 * 24) + align256((size_t)T * H / 32);
}

size_t prefill_packed_bytes(int num_slots, int H, int I) { return (size_t)num_slots * pk_slot_bytes(H, I); }

hipError_t launch_pack_weights(const ExpertStore& w, uint8_t* dst, hipStream_t s) {
  if (w.num_slots <= 0) return hipSuccess;
  const long threads = 64L * (2L * (w.I / 32) * pk_pairs(w.H) + (long)(w.H / 32) * pk_pairs(w.I));
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((threads + 255) / 256), (unsigned)w.num_slots), dim3(256), 0, s,
                     w, dst);
  return hipGetLastError();
}

hipError_t launch_prefill(const uint16_t* x, int T, int k, int E, const ExpertStore& w, const int32_t* e2s,
                          const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws,
                          hipStream_t s, const uint8_t* run, const uint8_t* packed) {
  const int H = w.H, I = w.I;
  if (H % 256 != 0 || I % 128 != 0) return hipErrorInvalidValue;
  const int ntw_gu = (I + GU_N - 1) / GU_N, ntw_dn = (H + DN_N - 1) / DN_N;
  const size_t P = (size_t)T * k, nm = max_mtiles(P);
  const size_t xq_b = P * H / 32 * 24, xs_b = P * H / 32;  // per sorted row (each token k times)
  const size_t hq_b = P * I / 32 * 24, hs_b = P * I / 32;
  if (xq_b >= kOob || hq_b >= kOob) return hipErrorInvalidValue;
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint8_t* xq = base;
  uint8_t* xs = xq + align256(xq_b);
  uint8_t* hq = xs + align256(xs_b);
  uint8_t* hs = hq + align256(hq_b);
  TileDesc* gu = reinterpret_cast<TileDesc*>(hs + align256(hs_b));
  TileDesc* dn = reinterpret_cast<TileDesc*>(reinterpret_cast<uint8_t*>(gu) +
                                             align256(nm * ntw_gu * sizeof(TileDesc)));
  SkBucket* sbk = reinterpret_cast<SkBucket*>(reinterpret_cast<uint8_t*>(dn) +
                                             align256(nm * ntw_dn * sizeof(TileDesc)));
  int32_t* counts = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(sbk) +
                                               align256(kMaxExperts * sizeof(SkBucket)));
  uint8_t* xq_t = reinterpret_cast<uint8_t*>(counts) + 256;  // token-major x blocks, then their scales
  uint8_t* xs_t = xq_t + align256((size_t)T * H / 32 * 24);
  const int nblk = T * (H / 32), nsw = (H / 128) * (int)((P + 63) / 64);  // sort_x: wavefronts
  hipLaunchKernelGGL(quant_x_kernel, dim3((nblk + kPT - 1) / kPT), dim3(kPT), 0, s, x, nblk, xq_t, xs_t);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_x_kernel, dim3((nsw + kPT / 64 - 1) / (kPT / 64)), dim3(kPT), 0, s, xq_t, xs_t, H, k, (int)P,
                     offsets, E, sorted_pair, xq, reinterpret_cast<uint32_t*>(xs));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(plan_kernel, dim3(kPlanGrid), dim3(kPT), 0, s, offsets, E, e2s, w.num_slots, ntw_gu, ntw_dn, run,
                     gu, dn, sbk, counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t nsk = min((size_t)E, P);  // small buckets at most
  const int gu_grid = (int)((nsk * (size_t)(I / 32) + 3) / 4), dn_grid = (int)((nsk * (size_t)(H / 64) + 3) / 4);
  if (packed)
    hipLaunchKernelGGL(gateup_skinny_kernel<true>, dim3(gu_grid), dim3(kPT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b,
                       (int)P, w, packed, sorted_pair, sbk, counts, hq, hs);
  else
    hipLaunchKernelGGL(gateup_skinny_kernel<false>, dim3(gu_grid), dim3(kPT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b,
                       (int)P, w, packed, sorted_pair, sbk, counts, hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (packed)
    hipLaunchKernelGGL(gateup_tile_kernel<true>, dim3(kGrid), dim3(kTilePT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b,
                       (int)P, w, packed, gu, counts, hq, hs);
  else
    hipLaunchKernelGGL(gateup_tile_kernel<false>, dim3(kGrid), dim3(kTilePT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b,
                       (int)P, w, packed, gu, counts, hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (packed)
    hipLaunchKernelGGL(down_skinny_kernel<true>, dim3(dn_grid), dim3(kPT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b,
                       (int)P, w, packed, sorted_pair, sbk, counts, y_pair);
  else
    hipLaunchKernelGGL(down_skinny_kernel<false>, dim3(dn_grid), dim3(kPT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b,
                       (int)P, w, packed, sorted_pair, sbk, counts, y_pair);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (packed)
    hipLaunchKernelGGL(down_tile_kernel<true>, dim3(kGrid), dim3(kTilePT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b,
                       (int)P, w, packed, sorted_pair, dn, counts, y_pair);
  else
    hipLaunchKernelGGL(down_tile_kernel<false>, dim3(kGrid), dim3(kTilePT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b,
                       (int)P, w, packed, sorted_pair, dn, counts, y_pair);
  return hipGetLastError();
}

}  // namespace moe
