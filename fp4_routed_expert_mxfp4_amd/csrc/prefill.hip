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
// A GEMM tile is 128 bucket rows x 256 weight rows over all of K, in chunks of
// 256 (eight 32-blocks, four MFMA K-steps).  The weights, the large operand,
// stream from memory straight into the registers of the one wavefront that
// uses them; the activations are staged once per chunk through LDS and read
// by all four wavefronts.  Workgroups are persistent: the tile list (bucket,
// weight tile, row tile -- row tiles of one weight tile adjacent, so they
// share that weight tile in L2) is split into eight contiguous ranges, one
// per XCD.
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

// The token-major blocks copied into the sorted chunk-major layout: one
// thread per (chunk c, sorted row p) reads its token's 96 B and scale word of
// the chunk and writes the two 48-byte records (consecutive threads write
// consecutive records) and the chunk's scale word.  Only the rows that the
// bucketing filled are read: sorted rows at or past offsets[E] (pairs whose
// expert id was out of range are in no bucket) hold no pair index, and a
// pair index outside [0, T*k) is skipped as well.
__global__ __launch_bounds__(kPT) void sort_x_kernel(const uint8_t* __restrict__ xq_t,
                                                     const uint8_t* __restrict__ xs_t, int H, int k, int P,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     const int32_t* __restrict__ sorted_pair,
                                                     uint8_t* __restrict__ xq, uint32_t* __restrict__ xs) {
  const int g = blockIdx.x * kPT + threadIdx.x;
  const int nch = H / 128;
  if (g >= P * nch) return;
  const int c = g / P, p = g - c * P;
  if (p >= offsets[E]) return;
  const int pair = sorted_pair[p];
  if (pair < 0 || pair >= P) return;
  const size_t t = (size_t)(pair / k);
  const uint2* src = reinterpret_cast<const uint2*>(xq_t + (t * (H / 32) + 4 * c) * 24);
  uint2 w[12];  // block b of the chunk = w[3b .. 3b+2]
#pragma unroll
  for (int i = 0; i < 12; ++i) w[i] = src[i];
#pragma unroll
  for (int h = 0; h < 2; ++h) {  // record of K-half h: block h, then block 2+h
    uint2* dst = reinterpret_cast<uint2*>(xq + q6_offset(p, 4 * c + h, P));
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      dst[i] = w[3 * h + i];
      dst[3 + i] = w[3 * (2 + h) + i];
    }
  }
  xs[(size_t)c * P + p] = *reinterpret_cast<const uint32_t*>(xs_t + t * (H / 32) + 4 * c);
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
// A tile is BM = 128 bucket rows x 4 * WN = 512 weight rows over all of K, in
// chunks of 128 (four 32-blocks, two K-steps of V_MFMA_SCALE_F32_32X32X64).
// Each wavefront owns WN = 128 weight rows (four 32-row B fragments) and all
// 128 bucket rows (four A fragments): 16 MFMAs per K-step into 16 x 16 fp32
// accumulators per lane.  Its weight rows are used by no other wavefront, so
// they go from memory straight into its registers; the MXFP6 activations are
// shared by the four wavefronts and staged once per chunk through a
// three-stage LDS ring with one barrier per chunk.  With three stages the
// first K-step of chunk c+1 is read from LDS while chunk c is multiplied (it
// was stored before the previous barrier), and the stage refilled during
// chunk c (with chunk c+2) was last read before that barrier.  The scale
// bytes of the tile are read once per window of TWIN chunks into LDS tables
// (row-contiguous loads: a per-chunk 4-byte load from every row would cost a
// cache-line request per row).

// A copy of v that the compiler cannot see through: per-lane index arithmetic
// derived from it is recomputed where it is used instead of being hoisted out
// of the persistent tile loop (hoisted, the table and epilogue addresses of a
// tile would hold well over a hundred registers for the whole kernel).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

constexpr int WN = 128;             // weight rows per wavefront (four fragments)
constexpr int NSTAGE = 3;           // A chunks held in LDS
constexpr int A_HS = BM * 48 + 64;  // LDS bytes per K-half region of an A chunk
constexpr int A_STAGE = 2 * A_HS;   // LDS bytes per A chunk
constexpr int TWIN = 40;            // scale-table window in chunks (160 blocks)
constexpr int TSW = TWIN + 1;       // words per table row (odd: a fragment's 32 rows hit 32 banks)

struct TileSmem {
  union {
    struct {
      uint8_t a[NSTAGE][A_STAGE];
      uint32_t sca[BM * TSW];     // A scale words of the tile's rows, [row][chunk of the window]
      uint32_t scb[4][WN * TSW];  // B scale words of each wavefront's 128 weight rows
    } k;
    float stage[BM * (GU_N + 1)];  // gate/up epilogue: h of the tile, fp32
  };
  int rowtok[BM];
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
};

// Half (rows 64 HALF .. 64 HALF + 63) of the B scale table of one wavefront:
// words [cw0, cw0 + TWIN) of those weight rows, read as 8-byte pairs (a row's
// scale bytes are contiguous and 8-byte aligned: K is a multiple of 256).
// Words past a row's end belong to the next row or lie past the resource's
// range (zeros); they are never used.  row_off(r): byte offset of table row r.
template <int HALF>
struct BTable {
  static constexpr int N = (WN / 2) * TWIN / 2 / 64;  // 8-byte loads per lane
  uint2 v[N];
  template <typename RowRes, typename RowOff>
  __device__ __forceinline__ void issue(RowRes res, RowOff row_off, int cw0, int lane) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = lane + 64 * i, row = 64 * HALF + idx / (TWIN / 2), pr = idx % (TWIN / 2);
      v[i] = bload8(res(row), row_off(row) + 4u * (uint32_t)(cw0 + 2 * pr));
    }
  }
  __device__ __forceinline__ void store(uint32_t* tab, int lane) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = lane + 64 * i, row = 64 * HALF + idx / (TWIN / 2), pr = idx % (TWIN / 2);
      tab[row * TSW + 2 * pr] = v[i].x;
      tab[row * TSW + 2 * pr + 1] = v[i].y;
    }
  }
};

// One A chunk in registers between its loads and its LDS store: the tile's two
// record runs (K-half 0, then 1; 128 rows x 48 B each) as 768 pieces of 16 B,
// piece t + 256 j in thread t.  Memory and LDS hold the runs in the same order.
struct AStage {
  uint4_t q[3];
};

struct ASrc {
  rsrc_t rc;
  uint32_t vc[3];    // this thread's pieces of chunk 0
  uint32_t cstride;  // bytes per chunk: both K-halves of all P rows
  // Rows past the bucket read other buckets' records (their outputs are never
  // stored and their scale words are zero); past the array's end they read zeros.
  __device__ __forceinline__ void init(const uint8_t* base, uint32_t bytes, int tid, int row0, int P) {
    rc = make_rsrc(base, bytes);
    cstride = 96u * (uint32_t)P;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int i = tid + kPT * j, h = i / (BM * 3);
      vc[j] = ((uint32_t)h * (uint32_t)P + (uint32_t)row0) * 48u + (uint32_t)(i - h * BM * 3) * 16u;
    }
  }
  __device__ __forceinline__ void load(int c, AStage& r) const {
#pragma unroll
    for (int j = 0; j < 3; ++j) r.q[j] = bload16(rc, vc[j] + (uint32_t)c * cstride);
  }
};

__device__ __forceinline__ void store_a(uint8_t* st, const AStage& r, int tid) {
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int i = tid + kPT * j, h = i / (BM * 3);
    *reinterpret_cast<uint4_t*>(st + h * A_HS + (i - h * BM * 3) * 16) = r.q[j];
  }
}

// The lane's A operand of K-step S of fragment f: 24 bytes at offset 24 S of
// the 48-byte record of row 32 f + r32 in K-half h (blocks 4c + h and 4c + 2 + h).
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

// One wavefront's weight rows for one chunk: each fragment's 32 rows as two
// loads of 16 rows x 64 contiguous bytes (lane l: row 16 j + l % 16, block
// l / 16 of the chunk); b_operands() moves them into MFMA order.
struct BChunk {
  uint4_t q[4][2];  // [fragment][row half]
};

struct BSrc {
  rsrc_t rc[4];    // codes of the matrix holding each fragment
  uint32_t vc[4];  // fragment row (lane % 16) offset + 16 * (lane / 16)
  uint32_t half;   // byte distance of fragment row 16 from row 0
  __device__ __forceinline__ void load(int c, BChunk& r) const {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 2; ++j) r.q[g][j] = bload16(rc[g], vc[g] + half * j + (uint32_t)c * 64u);
  }
};

// Chunk c of the tile (i = c - cw0 within the window): both K-steps, 32
// MFMAs.  af holds the chunk's K-step 0 fragments on entry and the next
// chunk's on return (read from stage nxt).  run == false multiplies nothing
// (a chunk past the last one of a pair).
__device__ __forceinline__ void tile_chunk(const TileSmem& sm, const uint8_t* cur, const uint8_t* nxt,
                                           const BChunk& bc, i8v (&af)[4], f16v (&acc)[4][4], int i, int wid,
                                           int r32, int h, bool run) {
  uint32_t sa[4], sb[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) sa[f] = sm.k.sca[(32 * f + r32) * TSW + i] >> (8 * h);
#pragma unroll
  for (int g = 0; g < 4; ++g) sb[g] = sm.k.scb[wid][(32 * g + r32) * TSW + i] >> (8 * h);
  i8v bop[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) b_operands(bc.q[g][0], bc.q[g][1], bop[g][0], bop[g][1]);
  i8v af1[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) af1[f] = read_afrag<1>(cur, f, r32, h);
  if (run) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[f], bop[g][0], acc[f][g], 2, 4, 0,
                                                                     (int)sa[f], 0, (int)sb[g]);
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) af[f] = read_afrag<0>(nxt, f, r32, h);
  if (run) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af1[f], bop[g][1], acc[f][g], 2, 4, 0,
                                                                     (int)(sa[f] >> 16), 0, (int)(sb[g] >> 16));
  }
}

// All K of one tile.  B chunk c+1 is loaded while chunk c is multiplied (two
// register sets, so the loop runs in pairs of chunks), A chunk c+2 is loaded
// into registers at the start of chunk c and stored into its LDS stage at the
// end.  Loads past the window's last chunk re-read it, so no load sits behind
// a branch.  tables(cw0) issues and stores the scale tables of a window; the
// barrier after the first A stages makes them visible.
template <typename Tables>
__device__ __forceinline__ void tile_k_loop(TileSmem& sm, f16v (&acc)[4][4], const ASrc& as, const BSrc& bs,
                                            int nch, int tid, Tables tables) {
  const int lane = tid & 63, wid = tid >> 6, r32 = lane & 31, h = lane >> 5;
  for (int cw0 = 0; cw0 < nch; cw0 += TWIN) {
    const int last = min(cw0 + TWIN, nch) - 1;
    if (cw0 > 0) __syncthreads();  // every wavefront is done with the previous window
    AStage a0, a1;
    as.load(cw0, a0);
    as.load(min(cw0 + 1, last), a1);
    BChunk b0, b1;
    bs.load(cw0, b0);
    tables(cw0);
    store_a(sm.k.a[0], a0, tid);
    store_a(sm.k.a[1], a1, tid);
    __syncthreads();
    i8v af[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) af[f] = read_afrag<0>(sm.k.a[0], f, r32, h);
    int s0 = 0;  // LDS stage of chunk c
    for (int c = cw0; c <= last; c += 2) {
      const int s1 = s0 == 2 ? 0 : s0 + 1, s2 = s1 == 2 ? 0 : s1 + 1;
      // The loads of each step are pinned ahead of its MFMAs (sched_barrier):
      // left to itself the scheduler sinks them next to their first use.
      {  // chunk c (always present)
        AStage an;
        as.load(min(c + 2, last), an);
        bs.load(min(c + 1, last), b1);
        __builtin_amdgcn_sched_barrier(0);
        tile_chunk(sm, sm.k.a[s0], sm.k.a[s1], b0, af, acc, c - cw0, wid, r32, h, true);
        store_a(sm.k.a[s2], an, tid);
        __syncthreads();
      }
      {  // chunk c + 1 (past the last chunk of an odd window: loads and stores only)
        AStage an;
        as.load(min(c + 3, last), an);
        bs.load(min(c + 2, last), b0);
        __builtin_amdgcn_sched_barrier(0);
        tile_chunk(sm, sm.k.a[s1], sm.k.a[s2], b1, af, acc, c + 1 - cw0, wid, r32, h, c + 1 <= last);
        store_a(sm.k.a[s0], an, tid);
        __syncthreads();
      }
      s0 = s2;
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
// rows past the end read as zeros) and its two B fragments come straight from
// memory into registers in MFMA order, in batches of four K-steps with the next
// batch in flight, and many wavefronts per CU keep the HBM stream full.


// Four K-steps (two 128-K chunks) of one wavefront: A block 2s+h of row r32
// (24 B); each B fragment's rows as two halves of 16 rows x 64 B per chunk
// (moved into MFMA order by b_operands when used); and the scale words of
// those 8 blocks.
struct SkRegs {
  uint2 a[4][3];
  uint4_t b[2][2][2];  // [chunk][fragment][row half]
};

// Scale words come from a per-wavefront LDS table read once per window of
// SKWIN chunks: rows 0-31 the unit's A rows, 32-63 and 64-95 its two weight
// fragments (whose scale bytes are contiguous).
constexpr int SKWIN = 20;
constexpr int SKW = SKWIN + 1;  // words per table row (odd: 32 rows hit 32 banks)

struct SkSrc {
  rsrc_t ra, rb[2];
  uint32_t va, vb[2];  // va: the lane's record (row r32, K-half h) in chunk 0; vb: row (lane%16) + 16 * (lane/16)
  uint32_t cstride;    // bytes per chunk of the A records
  uint32_t half;       // byte distance of fragment row 16 from row 0
  __device__ __forceinline__ void load(int n, SkRegs& r) const {
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // K-step s: chunk 2n + s/2, block 2(s%2) + h = bytes 24(s%2).. of the record
      const uint32_t o = va + (uint32_t)(2 * n + (s >> 1)) * cstride + 24u * (uint32_t)(s & 1);
#pragma unroll
      for (int j = 0; j < 3; ++j) r.a[s][j] = bload8(ra, o + 8u * j);
    }
    // the two chunks' 64-B halves of each row's 128-B line back to back
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int m = 0; m < 2; ++m) r.b[m][g][j] = bload16(rb[g], vb[g] + half * j + (uint32_t)(2 * n + m) * 64u);
  }
};

__device__ __forceinline__ void sk_mma(const SkRegs& r, f16v (&acc)[2], int nks, int h, const uint32_t* tab,
                                       int cw) {  // cw: the batch's first chunk within the window
  const int r32 = __lane_id() & 31;
  i8v bop[2][4];  // [fragment][K-step]
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int g = 0; g < 2; ++g) b_operands(r.b[m][g][0], r.b[m][g][1], bop[g][2 * m], bop[g][2 * m + 1]);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < nks) {
      const i8v a = i8v{(int)r.a[s][0].x, (int)r.a[s][0].y, (int)r.a[s][1].x, (int)r.a[s][1].y,
                        (int)r.a[s][2].x, (int)r.a[s][2].y, 0, 0};
      // low byte: the scale of block 2s+h
      const int sa = (int)((tab[r32 * SKW + cw + (s >> 1)] >> (8 * h)) >> (16 * (s & 1)));
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int sb = (int)((tab[(32 + 32 * g + r32) * SKW + cw + (s >> 1)] >> (8 * h)) >> (16 * (s & 1)));
        acc[g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[g][s], acc[g], 2, 4, 0, sa, 0, sb);
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

// All K of one unit: batches of four K-steps, the next batch's loads in flight
// while one is multiplied; pairs of batches alternate the two register sets.
// Loads past the last batch re-read it (never used): no load behind a branch.
// tables(cw0, ts) issues the scale-table loads of the window starting at chunk cw0.
template <typename TS, typename Tables>
__device__ __forceinline__ void sk_k_loop(const SkSrc& src, f16v (&acc)[2], int K, int h, uint32_t* tab,
                                          Tables tables) {
  const int nks_total = K / 64, nchunks = K / KC;
  const int lane = __lane_id();
  for (int cw0 = 0; cw0 < nchunks; cw0 += SKWIN) {
    const int b0 = cw0 / 2, last = (min(cw0 + SKWIN, nchunks) + 1) / 2 - 1;  // batches of this window
    TS ts;
    tables(cw0, ts);
    SkRegs r0, r1;
    src.load(b0, r0);
    ts.a.store(tab, lane);
    ts.b[0].store(tab + 32 * SKW, lane);
    ts.b[1].store(tab + 64 * SKW, lane);
    __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses complete in order
    for (int n = b0; n <= last; n += 2) {
      src.load(min(n + 1, last), r1);
      sk_mma(r0, acc, min(4, nks_total - 4 * n), h, tab, 2 * (n - b0));
      src.load(min(n + 2, last), r0);
      sk_mma(r1, acc, n + 1 > last ? 0 : min(4, nks_total - 4 * (n + 1)), h, tab, 2 * (n + 1 - b0));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The streaming kernels launch one wavefront per possible unit (four per
// workgroup); those past the plan's unit count exit at once, and the hardware
// dispatcher balances the rest.

__global__ __launch_bounds__(kPT, 2) void gateup_skinny_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, uint32_t xq_bytes, uint32_t xs_bytes, int P,
    ExpertStore w, const int32_t* __restrict__ sorted_pair, const SkBucket* __restrict__ sbk,
    const int32_t* __restrict__ counts, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ float stage[4][32 * 33];
  __shared__ uint32_t sktab[4][96 * SKW];
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
    src.vb[0] = src.vb[1] = (uint32_t)(32 * q + (lane & 15)) * wrow + 16u * (uint32_t)(lane >> 4);
    src.half = 16u * wrow;
    const rsrc_t xsr = make_rsrc(xs, xs_bytes);
    const rsrc_t sgr = make_rsrc(w.sg + (size_t)bk.slot * smat, (uint32_t)smat);
    const rsrc_t sur = make_rsrc(w.su + (size_t)bk.slot * smat, (uint32_t)smat);
    using TS = SkTables<ScaleCols<32, 64, SKWIN, SKW>>;
    auto tables = [&](int cw0, TS& ts) {
      ts.a.issue(xsr, cw0, lane, bk.row0, bk.cnt, P);
      ts.b[0].issue(sgr, cw0, lane, [&](int r) { return (uint32_t)(32 * q + r) * NBH; });
      ts.b[1].issue(sur, cw0, lane, [&](int r) { return (uint32_t)(32 * q + r) * NBH; });
    };
    f16v acc[2] = {f16v{}, f16v{}};
    sk_k_loop<TS>(src, acc, H, h, sktab[wid], tables);
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

__global__ __launch_bounds__(kPT, 2) void down_skinny_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, uint32_t hq_bytes, uint32_t hs_bytes, int P,
    ExpertStore w, const int32_t* __restrict__ sorted_pair, const SkBucket* __restrict__ sbk,
    const int32_t* __restrict__ counts, float* __restrict__ y) {
  __shared__ uint32_t sktab[4][96 * SKW];
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
      src.vb[g] = (uint32_t)(n0 + 32 * g + (lane & 15)) * wrow + 16u * (uint32_t)(lane >> 4);
    }
    src.half = 16u * wrow;
    const rsrc_t hsr = make_rsrc(hs, hs_bytes);
    const rsrc_t sdr = make_rsrc(w.sd + (size_t)bk.slot * smat, (uint32_t)smat);
    using TS = SkTables<ScaleRows<32, 64, SKWIN, SKW>>;
    auto tables = [&](int cw0, TS& ts) {
      ts.a.issue(hsr, cw0, lane, [&](int r) { return r < bk.cnt ? (uint32_t)(bk.row0 + r) * NBI : kOob; });
      ts.b[0].issue(sdr, cw0, lane, [&](int r) { return (uint32_t)(n0 + r) * NBI; });
      ts.b[1].issue(sdr, cw0, lane, [&](int r) { return (uint32_t)(n0 + 32 + r) * NBI; });
    };
    f16v acc[2] = {f16v{}, f16v{}};
    sk_k_loop<TS>(src, acc, I, h, sktab[wid], tables);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + h * 4 + (i & 3);
      if (row < bk.cnt) {
        float* yr = y + (size_t)sorted_pair[bk.row0 + row] * H + n0 + r32;
        yr[0] = acc[0][i];
        yr[32] = acc[1][i];
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

__global__ __launch_bounds__(kPT, 1) void gateup_tile_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, uint32_t xq_bytes, uint32_t xs_bytes, int P,
    ExpertStore w, const TileDesc* __restrict__ tiles, const int32_t* __restrict__ counts,
    uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ TileSmem sm;
  const int H = w.H, I = w.I, NBH = H / 32, NBI = I / 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, r32 = lane & 31, h = lane >> 5;
  const uint32_t wrow = (uint32_t)H / 2u;
  const size_t mat = (size_t)I * wrow, smat = (size_t)I * NBH;
  const int total = counts[0];
  for (TileWalk tw(total); tw.next < tw.end; tw.next += tw.step) {
    const TileDesc d = tiles[tw.next];
    if (d.slot < 0) continue;  // no stored expert: the down GEMM writes its rows as zeros
    __syncthreads();           // the previous tile's epilogue is done with the LDS
    const int j0 = d.ntile * GU_N;
    const int hc0 = j0 + 64 * wid;           // this wavefront's first h column
    const bool live = hc0 < I;               // inter % 256 == 128: the last tile is half wide
    ASrc as;
    as.init(xq, xq_bytes, tid, d.row0, P);
    BSrc bs;
    const rsrc_t rg = make_rsrc(w.wg + (size_t)d.slot * mat, (uint32_t)mat);
    const rsrc_t ru = make_rsrc(w.wu + (size_t)d.slot * mat, (uint32_t)mat);
    const uint32_t lrow = (uint32_t)(lane & 15) * wrow + 16u * (uint32_t)(lane >> 4);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bs.rc[g] = g < 2 ? rg : ru;
      bs.vc[g] = live ? (uint32_t)(hc0 + 32 * (g & 1)) * wrow + lrow : kOob;
    }
    bs.half = 16u * wrow;
    const rsrc_t xsr = make_rsrc(xs, xs_bytes);
    const rsrc_t sgr = make_rsrc(w.sg + (size_t)d.slot * smat, (uint32_t)smat);
    const rsrc_t sur = make_rsrc(w.su + (size_t)d.slot * smat, (uint32_t)smat);
    auto tables = [&](int cw0) {
      const int t = opaque(tid), l = t & 63;
      // table rows 0-63: gate rows hc0.., 64-127: the same up rows
      const auto off = [&](int r) { return live ? (uint32_t)(hc0 + (r & 63)) * (uint32_t)NBH : kOob; };
      ScaleCols<BM, kPT, TWIN, TSW> ta;
      BTable<0> t0;
      BTable<1> t1;
      ta.issue(xsr, cw0, t, d.row0, d.mrows, P);
      t0.issue([&](int) { return sgr; }, off, cw0, l);
      ta.store(sm.k.sca, t);
      t0.store(sm.k.scb[wid], l);
      t1.issue([&](int) { return sur; }, off, cw0, l);
      t1.store(sm.k.scb[wid], l);
    };
    f16v acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = f16v{};
    tile_k_loop(sm, acc, as, bs, H / KC, tid, tables);  // ends on a barrier
    // h = silu(g) * u into the staging buffer
    {
      const int t = opaque(tid), e32 = t & 31, eh = (t >> 5) & 1;
      float* st = sm.stage + (eh * 4) * (GU_N + 1) + 64 * (t >> 6) + e32;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            st[(32 * f + (r >> 2) * 8 + (r & 3)) * (GU_N + 1) + 32 * i] = swiglu_fast(acc[f][i][r], acc[f][2 + i][r]);
    }
    __syncthreads();
    // MXFP6 of each (row, 32-block) of the tile, written in sorted-row order
    const int nblk = min(GU_N, I - j0) / 32;
    for (int item = opaque(tid); item < BM * (GU_N / 32); item += kPT) {
      const int row = item % BM, blk = item / BM;
      if (row < d.mrows && blk < nblk) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = sm.stage[row * (GU_N + 1) + 32 * blk + i];
        uint32_t pk[6], sb;
        q6_block(v, pk, sb);
        const size_t grow = (size_t)(d.row0 + row);
        const int gblk = j0 / 32 + blk;
        uint2* dst = reinterpret_cast<uint2*>(hq + q6_offset(d.row0 + row, gblk, P));
        dst[0] = make_uint2(pk[0], pk[1]);
        dst[1] = make_uint2(pk[2], pk[3]);
        dst[2] = make_uint2(pk[4], pk[5]);
        hs[grow * NBI + gblk] = (uint8_t)sb;
      }
    }
  }
}

// ---- P2: down GEMM -> y_pair ---------------------------------------------------------
//
// Wavefront w of a tile owns output columns n0 + 128 w .. + 127 (four
// fragments of W_down rows); each lane stores its accumulators straight into
// the y_pair rows of the tile's pairs (32 consecutive columns of two rows per
// store).  In a last tile narrower than 512 columns (hidden % 512 == 256)
// wavefronts 2 and 3 load zeros and store nothing.

__global__ __launch_bounds__(kPT, 1) void down_tile_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, uint32_t hq_bytes, uint32_t hs_bytes, int P,
    ExpertStore w, const int32_t* __restrict__ sorted_pair, const TileDesc* __restrict__ tiles,
    const int32_t* __restrict__ counts, float* __restrict__ y) {
  __shared__ TileSmem sm;
  const int H = w.H, I = w.I, NBI = I / 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, r32 = lane & 31, h = lane >> 5;
  const uint32_t wrow = (uint32_t)I / 2u;
  const size_t mat = (size_t)H * wrow, smat = (size_t)H * NBI;
  const int total = counts[1];
  for (TileWalk tw(total); tw.next < tw.end; tw.next += tw.step) {
    const TileDesc d = tiles[tw.next];
    __syncthreads();
    if (tid < BM) sm.rowtok[tid] = tid < d.mrows ? sorted_pair[d.row0 + tid] : -1;
    __syncthreads();
    const int n0 = d.ntile * DN_N;
    const int nc0 = n0 + WN * wid;  // this wavefront's first output column
    const bool live = nc0 < H;
    if (d.slot < 0) {
      for (int i = tid; i < d.mrows * DN_N; i += kPT) {
        const int row = i / DN_N, col = i % DN_N;
        if (n0 + col < H) y[(size_t)sm.rowtok[row] * H + n0 + col] = 0.f;
      }
      continue;
    }
    ASrc as;
    as.init(hq, hq_bytes, tid, d.row0, P);
    BSrc bs;
    const rsrc_t rd = make_rsrc(w.wd + (size_t)d.slot * mat, (uint32_t)mat);
    const uint32_t lrow = (uint32_t)(lane & 15) * wrow + 16u * (uint32_t)(lane >> 4);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bs.rc[g] = rd;
      bs.vc[g] = live ? (uint32_t)(nc0 + 32 * g) * wrow + lrow : kOob;
    }
    bs.half = 16u * wrow;
    const rsrc_t hsr = make_rsrc(hs, hs_bytes);
    const rsrc_t sdr = make_rsrc(w.sd + (size_t)d.slot * smat, (uint32_t)smat);
    auto tables = [&](int cw0) {
      // A scales: hs is row-major [sorted row][I/32], so its words are read row by row
      const int t = opaque(tid), l = t & 63;
      const auto res = [&](int) { return sdr; };
      const auto off = [&](int r) { return live ? (uint32_t)(nc0 + r) * (uint32_t)NBI : kOob; };
      ScaleRows<BM, kPT, TWIN, TSW> ta;
      BTable<0> t0;
      BTable<1> t1;
      ta.issue(hsr, cw0, t, [&](int r) { return r < d.mrows ? (uint32_t)(d.row0 + r) * (uint32_t)NBI : kOob; });
      t0.issue(res, off, cw0, l);
      ta.store(sm.k.sca, t);
      t0.store(sm.k.scb[wid], l);
      t1.issue(res, off, cw0, l);
      t1.store(sm.k.scb[wid], l);
    };
    f16v acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = f16v{};
    tile_k_loop(sm, acc, as, bs, I / KC, tid, tables);
    if (live) {
      const int t = opaque(tid), e32 = t & 31, eh = (t >> 5) & 1;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        __builtin_amdgcn_sched_barrier(0);  // one fragment's stores at a time (register pressure)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * f + (r >> 2) * 8 + eh * 4 + (r & 3);
          if (row < d.mrows) {
            float* yr = y + (size_t)sm.rowtok[row] * H + nc0 + e32;
#pragma unroll
            for (int g = 0; g < 4; ++g) yr[32 * g] = acc[f][g][r];
          }
        }
      }
    }
  }
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

hipError_t launch_prefill(const uint16_t* x, int T, int k, int E, const ExpertStore& w, const int32_t* e2s,
                          const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws,
                          hipStream_t s, const uint8_t* run) {
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
  const int nblk = T * (H / 32), nq = (int)P * (H / 128);
  hipLaunchKernelGGL(quant_x_kernel, dim3((nblk + kPT - 1) / kPT), dim3(kPT), 0, s, x, nblk, xq_t, xs_t);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_x_kernel, dim3((nq + kPT - 1) / kPT), dim3(kPT), 0, s, xq_t, xs_t, H, k, (int)P,
                     offsets, E, sorted_pair, xq, reinterpret_cast<uint32_t*>(xs));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(plan_kernel, dim3(kPlanGrid), dim3(kPT), 0, s, offsets, E, e2s, w.num_slots, ntw_gu, ntw_dn, run,
                     gu, dn, sbk, counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t nsk = min((size_t)E, P);  // small buckets at most
  const int gu_grid = (int)((nsk * (size_t)(I / 32) + 3) / 4), dn_grid = (int)((nsk * (size_t)(H / 64) + 3) / 4);
  hipLaunchKernelGGL(gateup_skinny_kernel, dim3(gu_grid), dim3(kPT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b, (int)P,
                     w, sorted_pair, sbk, counts, hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gateup_tile_kernel, dim3(kGrid), dim3(kPT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b, (int)P, w,
                     gu, counts, hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(down_skinny_kernel, dim3(dn_grid), dim3(kPT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b, (int)P, w,
                     sorted_pair, sbk, counts, y_pair);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(down_tile_kernel, dim3(kGrid), dim3(kPT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b, (int)P, w,
                     sorted_pair, dn, counts, y_pair);
  return hipGetLastError();
}

}  // namespace moe
