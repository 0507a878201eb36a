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
constexpr int GU_N = 128;          // gate/up tile: 128 h columns = 128 gate + 128 up weight rows
constexpr int DN_N = 256;          // down tile: 256 output columns
constexpr int STAGE_S = GU_N + 1;  // fp32 words per row of the h staging buffer
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
// A workgroup computes a tile of BM bucket rows x 256 weight rows over all of
// K, in chunks of 128 (four 32-blocks, two MFMA 32x32x64 K-steps).  Each
// wavefront owns 64 weight rows (two 32-row B fragments) and all BM rows (four
// A fragments): 8 MFMAs per K-step.  The weight rows are not shared between
// wavefronts, so they go straight from memory into the wavefront's registers
// in MFMA order, three chunks ahead.  The MXFP6 activations are shared: staged
// once per chunk through LDS (double-buffered, one barrier per chunk).  The
// scale tables and the h staging buffer fill most of the LDS, so one
// workgroup runs per CU (one wavefront per SIMD).
//
// LDS layout of one A chunk: for each K-half h a region of BM rows x 48 B --
// blocks h and 2+h of the chunk, i.e. the lane's A operand for K-steps 0 and 1
// -- read as three 16-B loads per lane (lanes 48 B apart touch every bank
// once); then one scale word (4 bytes) per row.

constexpr int A_HS = BM * 48 + 64;  // LDS bytes per K-half region of an A chunk

struct ABuf {
  uint8_t codes[2 * A_HS];
};

// Scale bytes are read once per tile into LDS tables (a scale word -- the 4
// blocks of one chunk -- per row and chunk, for a window of SCWIN chunks):
// per-chunk loads of 4 bytes from every row would each cost a cache-line
// request.  The rows of a wavefront's weight fragment are consecutive, so
// their table loads read contiguous memory.
constexpr int SCWIN = 40;       // largest scale window in chunks (160 blocks)
constexpr int SCW = SCWIN + 1;  // words per table row (odd: a fragment's 32 rows hit 32 banks)

struct GemmSmem {
  union {
    ABuf a[2];
    float stage[BM * STAGE_S];
  };
  uint32_t sca[BM * SCW];      // A scale words of the tile's rows
  uint32_t scb[4][64 * SCW];   // B scale words of each wavefront's 64 weight rows
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

// The scale tables of one tile for a window of WIN chunks: A rows (all
// threads; AS is the loader of the A scale layout) and each wavefront's two
// 32-row weight fragments.
template <int WIN, typename AS>
struct TileScales {
  static constexpr int kWin = WIN;
  static_assert(WIN <= SCWIN, "scale window");
  AS a;
  ScaleRows<32, 64, WIN, SCW> b[2];
};

// Registers of one A chunk between its global loads and its LDS store: the
// tile's two records runs (K-half 0, then 1; 128 rows x 48 B each) as 768
// pieces of 16 B, piece t + 256j in thread t.  Memory and LDS hold the runs
// in the same order, so the store is a plain copy.
struct ARegs {
  uint4_t q[3];
};

struct ASrc {
  rsrc_t rc;
  uint32_t vc[3];     // this thread's pieces of chunk 0
  uint32_t cstride;   // bytes per chunk: both K-halves of all P rows
  __device__ __forceinline__ void load(int c, ARegs& r) const {
#pragma unroll
    for (int j = 0; j < 3; ++j) r.q[j] = bload16(rc, vc[j] + (uint32_t)c * cstride);
  }
};

__device__ __forceinline__ void store_a(ABuf& d, const ARegs& r, int tid) {
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int i = tid + kPT * j, h = i / (BM * 3);
    *reinterpret_cast<uint4_t*>(d.codes + h * A_HS + (i - h * BM * 3) * 16) = r.q[j];
  }
}

// A offsets of a tile whose rows are sorted rows row0.. of P.  Rows past the
// bucket read other buckets' records (their outputs are never stored, and
// their scale words are zero); past the array's end they read zeros.
__device__ __forceinline__ void a_offsets(ASrc& as, int tid, int row0, int P) {
  as.cstride = 96u * (uint32_t)P;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int i = tid + kPT * j, h = i / (BM * 3);
    as.vc[j] = ((uint32_t)h * (uint32_t)P + (uint32_t)row0) * 48u + (uint32_t)(i - h * BM * 3) * 16u;
  }
}

// One wavefront's B operand for one chunk.  Each fragment's 32 rows are
// loaded as two halves of 16 rows x 64 contiguous bytes (lane l: row 16j +
// l%16, block l/16 of the chunk), which touches half the cache lines of the
// MFMA order (32 rows x 32 B); b_operands() moves them into MFMA order with two
// lane swaps per dword when they are used.
struct BRegs {
  uint4_t q[2][2];  // [fragment][row half], as loaded
};

struct BSrc {
  rsrc_t rc[2];     // codes of fragment 0 and 1
  uint32_t vc[2];   // row (lane%16) offset + 16 * (lane/16)
  uint32_t half;    // byte distance of row 16 from row 0
  __device__ __forceinline__ void load(int c, BRegs& r) const {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 2; ++j) r.q[g][j] = bload16(rc[g], vc[g] + half * j + (uint32_t)c * 64u);
  }
};


// One chunk of MFMAs: A fragments from LDS (48 B per lane = both K-steps),
// B from registers.  With an empty chunk (nks == 0) nothing is multiplied.
__device__ __forceinline__ void mma_chunk(const ABuf& cur, const BRegs& b, const uint32_t* sca, const uint32_t* scb,
                                          int cw, f16v (&acc)[4][2], int nks, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
  if (nks == 0) return;
  uint4_t av[4][3];
  uint32_t asw[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint4_t* p = reinterpret_cast<const uint4_t*>(cur.codes + h * A_HS + (32 * f + r32) * 48);
    av[f][0] = p[0];
    av[f][1] = p[1];
    av[f][2] = p[2];
    asw[f] = sca[(32 * f + r32) * SCW + cw] >> (8 * h);
  }
  uint32_t bsw[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) bsw[g] = scb[(32 * g + r32) * SCW + cw] >> (8 * h);
  i8v bop[2][2];
#pragma unroll
  for (int g = 0; g < 2; ++g) b_operands(b.q[g][0], b.q[g][1], bop[g][0], bop[g][1]);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      // dwords 6s..6s+5 of the lane's 48 B are its block at K-step s
      const uint32_t* w = reinterpret_cast<const uint32_t*>(av[f]) + 6 * s;
      const i8v a = i8v{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], 0, 0};
      const int sa = (int)(asw[f] >> (16 * s));  // low byte: block 2s+h
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const i8v bb = bop[g][s];
        const int sb = (int)(bsw[g] >> (16 * s));
        acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, acc[f][g], 2, 4, 0, sa, 0, sb);
      }
    }
  }
}

// The K loop over all chunks of one tile.  A ring of PF register sets keeps
// the loads of chunks c+1..c+PF-1 in flight while chunk c is multiplied (the
// gathered activation rows come from the last-level cache, a long round
// trip); A chunk c+1 moves from its registers to LDS at the end of chunk c.
// The loop runs in rounds of PF steps; steps past the last chunk multiply
// nothing, loads past it re-read it and stores past it write a stage nothing
// reads again, so no load or store of the loop sits behind a branch.
constexpr int PF = 4;

struct ChunkRegs {
  ARegs a;
  BRegs b;
};

template <typename TS, typename Tables>
__device__ __forceinline__ void gemm_k_loop(GemmSmem& sm, f16v (&acc)[4][2], const ASrc& as, const BSrc& bs,
                                            int K, int tid, int lane, Tables tables) {
  constexpr int WIN = TS::kWin;
  const int nchunks = K / KC, wid = tid >> 6;
  for (int cw0 = 0; cw0 < nchunks; cw0 += WIN) {
    const int last = min(cw0 + WIN, nchunks) - 1;
    TS ts;
    tables(cw0, ts);
    ChunkRegs r[PF];
#pragma unroll
    for (int j = 0; j < PF - 1; ++j) {
      as.load(min(cw0 + j, last), r[j].a);
      bs.load(min(cw0 + j, last), r[j].b);
    }
    // the tables and A chunk 0, made visible by the barrier below
    ts.a.store(sm.sca, tid);
    ts.b[0].store(sm.scb[wid], lane);
    ts.b[1].store(sm.scb[wid] + 32 * SCW, lane);
    store_a(sm.a[0], r[0].a, tid);
    __syncthreads();
    for (int c0 = cw0; c0 <= last; c0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int c = c0 + j;
        ChunkRegs& ahead = r[(j + PF - 1) % PF];
        as.load(min(c + PF - 1, last), ahead.a);
        bs.load(min(c + PF - 1, last), ahead.b);
        mma_chunk(sm.a[(c - cw0) & 1], r[j].b, sm.sca, sm.scb[wid], c - cw0, acc, c > last ? 0 : 2, lane);
        store_a(sm.a[(c - cw0 + 1) & 1], r[(j + 1) % PF].a, tid);
        __syncthreads();
      }
    }
  }
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
      st[row * 33 + r32] = swiglu_f32(acc[0][i], acc[1][i]);
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
// Wavefront w's fragments are gate rows j0+32w.. and the up rows with the same
// index, so h = silu(g)*u is formed in its registers; its 32 h columns are
// exactly one MXFP6 block per row.

__global__ __launch_bounds__(kPT, 1) void gateup_mfma_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, uint32_t xq_bytes, uint32_t xs_bytes, int P,
    ExpertStore w, const int32_t* __restrict__ sorted_pair, const TileDesc* __restrict__ tiles,
    const int32_t* __restrict__ counts, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ GemmSmem sm;
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
    ASrc as;
    as.rc = make_rsrc(xq, xq_bytes);
    a_offsets(as, tid, d.row0, P);
    BSrc bs;
    {
      // wavefront wid: gate rows j0+32*wid.. (fragment 0) and the same up rows (fragment 1)
      const uint32_t jr = (uint32_t)(j0 + 32 * wid + r32);
      bs.rc[0] = make_rsrc(w.wg + (size_t)d.slot * mat, (uint32_t)mat);
      bs.rc[1] = make_rsrc(w.wu + (size_t)d.slot * mat, (uint32_t)mat);
      const uint32_t jl = (uint32_t)(j0 + 32 * wid + (lane & 15));
      bs.vc[0] = bs.vc[1] = jl * wrow + 16u * (uint32_t)(lane >> 4);
      bs.half = 16u * wrow;
    }
    const rsrc_t xsr = make_rsrc(xs, xs_bytes);
    const rsrc_t sgr = make_rsrc(w.sg + (size_t)d.slot * smat, (uint32_t)smat);
    const rsrc_t sur = make_rsrc(w.su + (size_t)d.slot * smat, (uint32_t)smat);
    const uint32_t jr0 = (uint32_t)(j0 + 32 * wid);
    using TS = TileScales<40, ScaleCols<BM, kPT, 40, SCW>>;
    auto tables = [&](int cw0, TS& ts) {
      ts.a.issue(xsr, cw0, tid, d.row0, d.mrows, P);
      ts.b[0].issue(sgr, cw0, lane, [&](int r) { return (jr0 + (uint32_t)r) * NBH; });
      ts.b[1].issue(sur, cw0, lane, [&](int r) { return (jr0 + (uint32_t)r) * NBH; });
    };
    f16v acc[4][2];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[f][g] = f16v{};
    gemm_k_loop<TS>(sm, acc, as, bs, H, tid, lane, tables);
    // h = silu(g) * u into the staging buffer (the K loop ended on a barrier)
    const int wcol = 32 * wid + r32;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * f + (i >> 2) * 8 + h * 4 + (i & 3);
        sm.stage[row * STAGE_S + wcol] = swiglu_f32(acc[f][0][i], acc[f][1][i]);
      }
    __syncthreads();
    // MXFP6 of each (row, 32-block) of the tile, written in sorted-row order
    for (int item = tid; item < BM * (GU_N / 32); item += kPT) {
      const int row = item % BM, blk = item / BM;
      if (row < d.mrows) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = sm.stage[row * STAGE_S + 32 * blk + i];
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

__global__ __launch_bounds__(kPT, 1) void down_mfma_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, uint32_t hq_bytes, uint32_t hs_bytes, int P,
    ExpertStore w, const int32_t* __restrict__ sorted_pair, const TileDesc* __restrict__ tiles,
    const int32_t* __restrict__ counts, float* __restrict__ y) {
  __shared__ GemmSmem sm;
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
    if (d.slot < 0) {
      for (int i = tid; i < d.mrows * DN_N; i += kPT) {
        const int row = i / DN_N, col = i % DN_N;
        y[(size_t)sm.rowtok[row] * H + n0 + col] = 0.f;
      }
      continue;
    }
    ASrc as;
    as.rc = make_rsrc(hq, hq_bytes);
    a_offsets(as, tid, d.row0, P);
    BSrc bs;
    {
      // wavefront wid: output rows n0+64*wid+32g.. (fragment g)
      const rsrc_t rc = make_rsrc(w.wd + (size_t)d.slot * mat, (uint32_t)mat);
      const rsrc_t rs = make_rsrc(w.sd + (size_t)d.slot * smat, (uint32_t)smat);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t nr = (uint32_t)(n0 + 64 * wid + 32 * g);
        bs.rc[g] = rc;
        bs.vc[g] = (nr + (uint32_t)(lane & 15)) * wrow + 16u * (uint32_t)(lane >> 4);
      }
      bs.half = 16u * wrow;
      (void)rs;
    }
    const rsrc_t hsr = make_rsrc(hs, hs_bytes);
    const rsrc_t sdr = make_rsrc(w.sd + (size_t)d.slot * smat, (uint32_t)smat);
    const uint32_t nr0 = (uint32_t)(n0 + 64 * wid);
    using TS = TileScales<20, ScaleRows<BM, kPT, 20, SCW>>;
    auto tables = [&](int cw0, TS& ts) {
      ts.a.issue(hsr, cw0, tid, [&](int r) { return r < d.mrows ? (uint32_t)(d.row0 + r) * NBI : kOob; });
#pragma unroll
      for (int g = 0; g < 2; ++g)
        ts.b[g].issue(sdr, cw0, lane, [&](int r) { return (nr0 + 32u * g + (uint32_t)r) * NBI; });
    };
    f16v acc[4][2];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[f][g] = f16v{};
    gemm_k_loop<TS>(sm, acc, as, bs, I, tid, lane, tables);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      __builtin_amdgcn_sched_barrier(0);  // one fragment's stores at a time (register pressure)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * f + (i >> 2) * 8 + h * 4 + (i & 3);
        if (row < d.mrows) {
          float* yr = y + (size_t)sm.rowtok[row] * H + n0 + 64 * wid + r32;
          yr[0] = acc[f][0][i];
          yr[32] = acc[f][1][i];
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
         align256(P * I / 32) + align256(nm * (I / GU_N) * sizeof(TileDesc)) +
         align256(nm * (H / DN_N) * sizeof(TileDesc)) + align256(kMaxExperts * sizeof(SkBucket)) + 256 +
         align256((size_t)T * H / 32 * 24) + align256((size_t)T * H / 32);
}

hipError_t launch_prefill(const uint16_t* x, int T, int k, int E, const ExpertStore& w, const int32_t* e2s,
                          const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws,
                          hipStream_t s, const uint8_t* run) {
  const int H = w.H, I = w.I;
  if (H % DN_N != 0 || I % GU_N != 0) return hipErrorInvalidValue;
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
                                             align256(nm * (I / GU_N) * sizeof(TileDesc)));
  SkBucket* sbk = reinterpret_cast<SkBucket*>(reinterpret_cast<uint8_t*>(dn) +
                                             align256(nm * (H / DN_N) * sizeof(TileDesc)));
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
  hipLaunchKernelGGL(plan_kernel, dim3(kPlanGrid), dim3(kPT), 0, s, offsets, E, e2s, w.num_slots, I / GU_N, H / DN_N, run,
                     gu, dn, sbk, counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t nsk = min((size_t)E, P);  // small buckets at most
  const int gu_grid = (int)((nsk * (size_t)(I / 32) + 3) / 4), dn_grid = (int)((nsk * (size_t)(H / 64) + 3) / 4);
  hipLaunchKernelGGL(gateup_skinny_kernel, dim3(gu_grid), dim3(kPT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b, (int)P,
                     w, sorted_pair, sbk, counts, hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gateup_mfma_kernel, dim3(kGrid), dim3(kPT), 0, s, xq, xs, (uint32_t)xq_b, (uint32_t)xs_b, (int)P, w,
                     sorted_pair, gu, counts, hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(down_skinny_kernel, dim3(dn_grid), dim3(kPT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b, (int)P, w,
                     sorted_pair, sbk, counts, y_pair);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(down_mfma_kernel, dim3(kGrid), dim3(kPT), 0, s, hq, hs, (uint32_t)hq_b, (uint32_t)hs_b, (int)P, w,
                     sorted_pair, dn, counts, y_pair);
  return hipGetLastError();
}

}  // namespace moe
