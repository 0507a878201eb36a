// Multi-token decode FFN over MXFP4 experts on gfx950 bf16 MFMA.
//
// Decode with more than one token (a small decode batch, the draft tokens a
// speculative step verifies) keeps the decode arithmetic: x stays bf16 and h
// keeps the precision of fp32, as the one-token kernels do ("Fast single-box
// DeepSeek v4.1 Flash runtime", "Conventions": decode is judged against
// unquantised activations).  A bucket -- the rows routed to one expert, at
// most one per token -- is a skinny GEMM, so groups of 16 of its rows are the
// M dimension of V_MFMA_F32_16X16X32_BF16 and 16 weight rows its N dimension:
//
//  * weights: e2m1 codes decoded to bf16 with the block's UE8M0 scale folded
//    in (v_cvt_scalef32_pk_bf16_fp4).  Exact while the scaled value is a
//    normal bf16 (block scales of 2^-125 and up): an e2m1 value has two
//    significant bits and the scale is a power of two.
//  * x: bf16 as given; every product is exact in fp32 and the MFMA sums in fp32.
//  * h: silu(g) * u is stored as two bf16 planes, hi = rne(h) and
//    lo = rne(h - hi); the down projection multiplies both (two MFMAs per
//    K-step), so h enters it with a relative error of at most 2^-18.
//
// Kernel G (gate/up): a unit is (bucket, group of 16 bucket rows, 32 h
//   columns): one A fragment (the rows' x, rows past the bucket's end read as
//   zeros) against four B fragments (16 gate rows, 16 more, and the same rows
//   of W_up).
// Kernel D (down): a unit is (bucket, group of 16 rows, 64 output columns):
//   A = the rows' h planes, B = four fragments of 16 W_down rows; y_pair rows
//   are written once.
//
// A unit belongs to one workgroup; its four wavefronts take fixed quarters of
// K and add their partial sums in LDS in wavefront order.  A row's result is
// therefore one fixed fp32 expression of its own inputs: bit-identical
// whichever other rows share its bucket and batch.
//
// K runs in chunks of 128 (four 32-blocks).  In the MFMA's operand order a B
// fragment's chunk is lane l: block 4c + l/16 of row l%16 (16 rows x 64
// contiguous bytes); K-step t takes dword t (codes 8t..8t+7) of that block, and
// A's lane the same 8 values of x (or h) of its row.  The down kernels load B
// in that order, one chunk at a time.  The gate/up kernels take chunk pairs
// and load each fragment's pair as two loads of 8 rows x 128 bytes (lane l:
// row 8j + l/8, bytes 16 (l%8) of the pair), a shape the memory pipeline
// streams faster than 16 half lines, and move the pieces into operand order
// through the wavefront's own LDS area.  The scale bytes of a window of chunks
// are read once per wavefront into an LDS table (contiguous row reads); the
// next chunks' loads are in flight while the current ones are multiplied.  The
// workgroups are persistent and walk the units grid-stride.
#include "common.cuh"
#include "kernels.h"
#include "route_core.cuh"

#include <type_traits>

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kMtThreads = 256;   // four wavefronts: the four quarters of a unit's K
constexpr int kMtGridGU = 512;    // persistent workgroups of the gate/up kernel (two per CU)
constexpr int kMtGridDN = 512;    // and of the down kernel (two per CU)
constexpr int kMtWin = 20;        // chunks per scale window (80 blocks; even: whole chunk pairs)
constexpr int kMtW = kMtWin + 1;  // words per table row (odd: 16 rows hit 16 banks)
constexpr int kMtRows = 16;       // bucket rows per unit (the MFMA's M)
constexpr int kMtFrags = 4;       // 16-row weight fragments per unit

// The bucket list and, per bucket, the prefix of its groups of kMtRows rows: bucket b
// owns units [tiles * G[b], tiles * G[b+1]), its groups of one column tile
// adjacent (they read the same weights).
struct MtPlan {
  Buckets bk;
  int G[kMaxExperts + 1];

  __device__ void build(const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ run) {
    build_buckets(offsets, E, bk, run);
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x, n = bk.n;
      constexpr int CH = kMaxExperts / 64;
      int v[CH], s = 0;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int b = lane * CH + i;
        v[i] = b < n ? (bk.cnt[b] + kMtRows - 1) / kMtRows : 0;
        s += v[i];
      }
      int incl = s;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      int pos = incl - s;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        G[lane * CH + i] = pos;
        pos += v[i];
      }
      if (lane == 63) G[kMaxExperts] = incl;
    }
    __syncthreads();
  }

  __device__ int groups() const { return G[kMaxExperts]; }

  // unit u -> bucket b, row group mg, column tile q
  __device__ void locate(int u, int tiles, int& b, int& mg, int& q) const {
    const int gi = u / tiles;
    int lo = 0, hi = bk.n;  // G[lo] <= gi < G[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (G[mid] <= gi) lo = mid; else hi = mid;
    }
    b = lo;
    const int ng = G[b + 1] - G[b], local = u - tiles * G[b];
    q = local / ng;
    mg = local - q * ng;
  }
};

// Eight e2m1 codes (one dword, code 2i in the low nibble of byte i) times the
// block scale, as eight bf16.
__device__ __forceinline__ bf16x8_t dq8(uint32_t w, float s) {
  const uint4_t u = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3))};
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// A copy of v the compiler cannot see through: per-lane addresses derived from
// it are recomputed where used instead of being hoisted out of a persistent
// loop, where they would hold registers for its whole length.
__device__ __forceinline__ int opaque_lane(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// CH consecutive chunks of one unit (one or two): A (per chunk and plane the
// lane's 64 B of block 4c+g) and the unit's NF B fragments.  CH = 1 (down):
// b[0][f] is fragment f in operand order (lane: 16 B = block 4c+g of row
// l%16).  CH = 2 (gate/up): b[j][f] is the j-th 8-row load of fragment f's
// chunk pair (lane l: row 8j + l/8, bytes 16 (l%8) of the pair), put in
// operand order through LDS (mt_stage, mt_fetch).
template <int PLANES, int CH, int NF>
struct MtRegs {
  uint4_t a[CH][PLANES][4];  // [chunk][plane][K-step]
  uint4_t b[CH][NF];         // CH = 1: [0][fragment]; CH = 2: [load][fragment]
};

// A chunk at or past `end` reads as zeros: its offsets get kOob, past every
// range (real offsets stay below 2^31).
template <int PLANES, int NF>
struct MtSrc {
  rsrc_t ra, rb[NF];
  uint32_t va;        // the lane's A row + 64 * g (kOob past the bucket's end)
  uint32_t plane;     // byte distance of the A planes
  uint32_t vb[NF];    // CH = 1: fragment row l%16, + 16 g; CH = 2: fragment row l/8, + 16 (l%8)
  uint32_t row8;      // CH = 2: bytes from a weight row to the row 8 below
  // A of chunks c .. c+CH-1
  template <int CH>
  __device__ __forceinline__ void load_a(int c, int end, MtRegs<PLANES, CH, NF>& r) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t off = c + i < end ? 0u : kOob;
#pragma unroll
      for (int p = 0; p < PLANES; ++p)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          r.a[i][p][t] = bload16(ra, (va + p * plane + (uint32_t)(c + i) * 256u + 16u * t) | off);
    }
  }
  // B of chunk c in operand order (CH = 1)
  __device__ __forceinline__ void load_b1(int c, int end, MtRegs<PLANES, 1, NF>& r) const {
    const uint32_t off = c < end ? 0u : kOob;
#pragma unroll
    for (int f = 0; f < NF; ++f) r.b[0][f] = bload16(rb[f], (vb[f] + (uint32_t)c * 64u) | off);
  }
  // B of chunks c, c+1 in 8-row loads (CH = 2); the lane's 16 B lie in chunk c + (l%8)/4
  __device__ __forceinline__ void load_b2(int c, int end, MtRegs<PLANES, 2, NF>& r) const {
    const uint32_t ob = c + ((__lane_id() >> 2) & 1) < end ? 0u : kOob;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 2; ++j) r.b[j][f] = bload16(rb[f], (vb[f] + (uint32_t)j * row8 + (uint32_t)c * 64u) | ob);
  }
};

// The chunk pair of the NF fragments (b: MtRegs<., 2, NF>::b) is written to
// the wavefront's LDS area scr (NF * 2 KB) and read back in operand order,
// chunk by chunk.  Fragment f has 2 KB at 2048 f: chunk i at 1024 i, the 16 B
// of operand lane t at slot t ^ (4i + t/16) ^ 8 (t & 1).  The swizzle keeps
// the 16 lanes of a write (two rows, all eight pieces) and of a read (16 rows)
// on 16 distinct 16-byte bank groups.  A wavefront's LDS accesses complete in
// order, so the area is reused by the next pair without a wait.
template <int NF>
__device__ __forceinline__ void mt_stage(const uint4_t (&b)[2][NF], uint8_t* scr) {
  const int lane = __lane_id(), rr = lane >> 3, p = lane & 7, i = p >> 2, g = p & 3;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int slot = ((8 * j + rr + 16 * g) ^ p) ^ (8 * (rr & 1));
#pragma unroll
    for (int f = 0; f < NF; ++f) *reinterpret_cast<uint4_t*>(scr + f * 2048 + i * 1024 + slot * 16) = b[j][f];
  }
}

// chunk ci of the staged pair: bq[f] = fragment f in operand order
template <int NF>
__device__ __forceinline__ void mt_fetch(const uint8_t* scr, int ci, uint4_t (&bq)[NF]) {
  const int lane = __lane_id(), tg = lane >> 4, odd = 8 * (lane & 1);
#pragma unroll
  for (int f = 0; f < NF; ++f)
    bq[f] = *reinterpret_cast<const uint4_t*>(scr + f * 2048 + ci * 1024 + ((lane ^ (4 * ci + tg)) ^ odd) * 16);
}

// The MFMAs of one chunk: 4 K-steps x NF fragments x PLANES, B (bq) in operand
// order.  The lane's scale is byte g of its row's table word in column col.
// Every output column's sum depends only on its own fragment.
template <int PLANES, int NF>
__device__ __forceinline__ void mt_mma_chunk(const uint4_t (&a)[PLANES][4], const uint4_t (&bq)[NF],
                                             f4v (&acc)[NF], const uint32_t* tab, int col, int q16, int g) {
  float sc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) sc[f] = ue8m0_to_f32((tab[(16 * f + q16) * kMtW + col] >> (8 * g)) & 0xFFu);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const bf16x8_t bw = dq8(bq[f][t], sc[f]);
#pragma unroll
      for (int p = 0; p < PLANES; ++p)
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[p][t]), bw, acc[f], 0, 0, 0);
    }
}

// Scale tables of a unit's window (table row 16 f + r: row r of fragment f).
// Gate/up: the gate rows' table then the up rows' (8 NF rows each); down: one
// table of 16 NF rows.
template <int NF>
struct MtTabGU {
  ScaleRows<8 * NF, 64, kMtWin, kMtW> t[2];
  __device__ __forceinline__ void store(uint32_t* tab, int lane) const {
    t[0].store(tab, lane);
    t[1].store(tab + 8 * NF * kMtW, lane);
  }
};
template <int NF>
struct MtTabDN {
  ScaleRows<16 * NF, 64, kMtWin, kMtW> t;
  __device__ __forceinline__ void store(uint32_t* tab, int lane) const { t.store(tab, lane); }
};

// The chunks [cb, ce) of one unit (down): windows of kMtWin chunks; in a
// window two register sets of one chunk alternate, the next chunk's loads in
// flight while one is multiplied.  A chunk past the window's end is skipped;
// the loads are unconditional (past the end they read zeros) and pinned ahead
// of the MFMAs they overlap.  tables(cw0, ts) issues the scale loads of the
// window starting at chunk cw0.
template <typename TS, int PLANES, int NF, typename Tables>
__device__ __forceinline__ void mt_k_loop(const MtSrc<PLANES, NF>& src, f4v (&acc)[NF], int cb, int ce,
                                          uint32_t* tab, Tables tables) {
  const int lane = __lane_id(), q16 = lane & 15, g = lane >> 4;
  for (int cw0 = cb; cw0 < ce; cw0 += kMtWin) {
    const int end = min(cw0 + kMtWin, ce), last = end - 1;
    TS ts;
    tables(cw0, ts);
    MtRegs<PLANES, 1, NF> r[2];
    auto load = [&](int c, MtRegs<PLANES, 1, NF>& dst) {
      src.load_b1(min(c, last), c < end ? end : 0, dst);
      src.template load_a<1>(min(c, last), c < end ? end : 0, dst);
    };
    load(cw0, r[0]);
    ts.store(tab, lane);
    __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses complete in order
    for (int c0 = cw0; c0 < end; c0 += 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = c0 + j;
        load(c + 1, r[j ^ 1]);
        __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads go out before these MFMAs
        if (j == 0 || c < end) mt_mma_chunk(r[j].a[0], r[j].b[0], acc, tab, c - cw0, q16, g);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The chunks [cb, ce) of one unit in chunk pairs (gate/up), B two pairs ahead
// and A one pair ahead: sets n = chunks cw0 + 2n, +1 of a window.  Issue
// order: A(0), B(0), B(1), then per set n, once B(n) is staged in LDS:
// A(n+1), B(n+2).  Loads complete in order, so set n waits for A(n) and B(n)
// only, with B(n+1) still in flight, and the MFMAs of set n overlap two sets'
// weight loads.  Every load and staging is unconditional (past the window's
// end they read zeros) so each wait covers one set; a set wholly past the end
// is not multiplied, the zero second chunk of a set that straddles it is.
template <typename TS, int PLANES, int NF, typename Tables>
__device__ __forceinline__ void mt_k_loop_deep(const MtSrc<PLANES, NF>& src, f4v (&acc)[NF], int cb, int ce,
                                               uint32_t* tab, uint8_t* scr, Tables tables) {
  const int lane = __lane_id(), q16 = lane & 15, g = lane >> 4;
  for (int cw0 = cb; cw0 < ce; cw0 += kMtWin) {
    const int end = min(cw0 + kMtWin, ce), last = end - 1;
    TS ts;
    tables(cw0, ts);
    MtRegs<PLANES, 2, NF> r[2];  // r[i].a: A of set n (n % 2 == i); r[i].b: raw B of set n, then n + 2
    auto load_a = [&](int n, MtRegs<PLANES, 2, NF>& dst) {
      const int c = cw0 + 2 * n;
      src.template load_a<2>(min(c, last), c < end ? end : 0, dst);
    };
    auto load_b = [&](int n, MtRegs<PLANES, 2, NF>& dst) {
      const int c = cw0 + 2 * n;
      src.load_b2(min(c, last), c < end ? end : 0, dst);
    };
    load_a(0, r[0]);
    load_b(0, r[0]);
    load_b(1, r[1]);
    ts.store(tab, lane);
    __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses complete in order
    for (int n0 = 0; cw0 + 2 * n0 < end; n0 += 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + j, c = cw0 + 2 * n;
        mt_stage<NF>(r[j].b, scr);
        load_a(n + 1, r[j ^ 1]);
        load_b(n + 2, r[j]);
        __builtin_amdgcn_sched_barrier(0);  // the next loads go out before these MFMAs
        if (j == 0 || c < end) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {  // a chunk past the window's end takes column `last`'s scales
            uint4_t bq[NF];
            mt_fetch<NF>(scr, i, bq);
            mt_mma_chunk(r[j].a[i], bq, acc, tab, min(c + i, last) - cw0, q16, g);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// A workgroup's gate/up units as one stream (units whose K quarter fits one
// scale window): the loads that mt_k_loop_deep issues past a unit's end (its
// sets nsets, nsets + 1) are the next unit's first sets instead, and the next
// unit's scale table is loaded before this unit's epilogue, so the next
// unit's first weights arrive while this one's partial sums are added.  The
// chunks, their order and the MFMA sequence of every unit are those of
// mt_k_loop_deep.
template <int NF>
struct GuUnit {
  int live;            // a unit to compute (otherwise every load reads zeros)
  int u;               // its index
  rsrc_t rg, ru;       // its gate and up codes
  rsrc_t sg, su;       // and their scale bytes
  uint32_t boff;       // byte offset of its first weight row (8 NF q rows)
  uint32_t srow;       // its first weight row
  int pair;            // the lane's A row as make() found it (its A offset is taken at first use)
  int info[5];         // what the epilogue needs
};

// make(u, U): the first live unit at or after u (stepping by stride), or
// U.live = 0; va_of(U.pair): the lane's A offset (row + 64 g, kOob for none),
// taken where the first A loads go out so that a row index make() loaded is
// not waited for earlier; epi(U, acc): the unit's epilogue.  x: the A rows'
// resource.
// vb0[f]: the lane's byte offset in the fragment-row pattern (row f*16 % 8NF/2
// + l/8, + 16 (l%8)) without the unit's offset.
template <int NF, typename Make, typename VaOf, typename Epi>
__device__ __forceinline__ void mt_gu_stream(int u0, int stride, int cb, int ce, int NB, uint32_t row8, rsrc_t x,
                                             uint32_t* tab, uint8_t* scr, Make make, VaOf va_of, Epi epi) {
  constexpr int NG = NF / 2;
  const int lane = __lane_id(), q16 = lane & 15, g = lane >> 4;
  // sets of the quarter, padded to an even count (a padded set reads zeros and
  // is not multiplied) so that every unit starts in register set 0
  const int nreal = (ce - cb + 1) >> 1, nsets = (nreal + 1) & ~1, last = ce - 1;
  const uint32_t half = ((uint32_t)lane >> 2) & 1u;  // the lane's 16 B of a pair lie in chunk c + half
  uint32_t vb0[NG];
#pragma unroll
  for (int f = 0; f < NG; ++f) vb0[f] = (uint32_t)(16 * f + (lane >> 3)) * (row8 / 8u) + 16u * (uint32_t)(lane & 7);
  auto tables = [&](const GuUnit<NF>& U, MtTabGU<NF>& ts) {
    const int t = opaque_lane(lane);
    ts.t[0].issue(U.sg, cb, t, [&](int r) { return U.live ? (U.srow + (uint32_t)r) * (uint32_t)NB : kOob; });
    ts.t[1].issue(U.su, cb, t, [&](int r) { return U.live ? (U.srow + (uint32_t)r) * (uint32_t)NB : kOob; });
  };
  // A of set n (chunks cb + 2n, +1) from row offset va (kOob: zeros)
  auto load_a = [&](uint32_t va, int n, MtRegs<1, 2, NF>& dst) {
    const int c = cb + 2 * n;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = c + i < ce ? 0u : kOob;
#pragma unroll
      for (int t = 0; t < 4; ++t) dst.a[i][0][t] = bload16(x, (va + (uint32_t)(c + i) * 256u + 16u * t) | off);
    }
  };
  // B of set n of the unit with codes rg, ru at boff (live == 0: zeros)
  auto load_b = [&](rsrc_t rg, rsrc_t ru, uint32_t boff, int live, int n, MtRegs<1, 2, NF>& dst) {
    const int c = cb + 2 * n;
    const uint32_t ob = live && c + (int)half < ce ? 0u : kOob;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        // non-temporal: a unit's weight rows are read once (verify16 173.3 -> 161.8 us); the
        // same policy on the down loads measured slower
        dst.b[j][f] = bload16_nt(f < NG ? rg : ru, (vb0[f % NG] + boff + (uint32_t)j * row8 + (uint32_t)c * 64u) | ob);
  };
  GuUnit<NF> U, N;
  make(u0, U);
  if (!U.live) return;
  MtTabGU<NF> ts;
  tables(U, ts);
  MtRegs<1, 2, NF> r[2];
  load_a(va_of(U.pair), 0, r[0]);
  load_b(U.rg, U.ru, U.boff, 1, 0, r[0]);
  load_b(U.rg, U.ru, U.boff, 1, 1, r[1]);
  for (;;) {
    ts.store(tab, opaque_lane(lane));  // waits for the table's loads, issued after this unit's first sets
    __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses complete in order
    make(U.u + stride, N);  // after the wait: its row-index load is not waited for here
    const uint32_t uva = va_of(U.pair);
    f4v acc[NF] = {};
    // set n: B(n) staged, A(n + 1) and B(n + 2) issued (this unit's, or with
    // NEXT the next unit's first sets), then the MFMAs of set n
    auto step = [&](auto J, auto NA, auto NB, int n) {
      constexpr int j = decltype(J)::value;
      constexpr bool na = decltype(NA)::value, nb = decltype(NB)::value;
      const int c = cb + 2 * n;
      mt_stage<NF>(r[j].b, scr);
      if constexpr (na) load_a(va_of(N.pair), n + 1 - nsets, r[j ^ 1]);
      else load_a(uva, n + 1, r[j ^ 1]);
      if constexpr (nb) load_b(N.rg, N.ru, N.boff, N.live, n + 2 - nsets, r[j]);
      else load_b(U.rg, U.ru, U.boff, 1, n + 2, r[j]);
      __builtin_amdgcn_sched_barrier(0);  // the next loads go out before these MFMAs
      if (n < nreal) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {  // a chunk past the quarter's end takes column `last`'s scales
          uint4_t bq[NF];
          mt_fetch<NF>(scr, i, bq);
          mt_mma_chunk(r[j].a[i], bq, acc, tab, min(c + i, last) - cb, q16, g);
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using F = std::false_type;
    using T = std::true_type;
    for (int n = 0; n + 2 < nsets; n += 2) {
      step(I0{}, F{}, F{}, n);
      step(I1{}, F{}, F{}, n + 1);
    }
    step(I0{}, F{}, T{}, nsets - 2);  // B of the next unit's set 0
    step(I1{}, T{}, T{}, nsets - 1);  // its A of set 0 and B of set 1
    __builtin_amdgcn_sched_barrier(0);  // the table's loads after the last MFMAs (their registers)
    tables(N, ts);
    epi(U, acc);
    if (!N.live) break;
    U = N;
  }
}

// The four wavefronts of a workgroup take fixed quarters of a unit's K
// (chunks [w*nch/4, (w+1)*nch/4)); their partial sums meet in LDS and are
// added in wavefront order, so every output is the same fp32 expression
// whatever the batch around it.  part: the wavefront's own table area, free
// once its K loop is done.
template <int NF>
__device__ __forceinline__ void mt_part_store(float* part, const f4v (&acc)[NF], int lane) {
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) part[(4 * f + v) * 64 + lane] = acc[f][v];
}

// fragment f, accumulator v of the whole unit: partial 0 + 1 + 2 + 3
template <int NF>
__device__ __forceinline__ float mt_part_sum(const uint32_t (*tabs)[16 * NF * kMtW], int f, int v, int lane) {
  const int i = (4 * f + v) * 64 + lane;
  float s = __uint_as_float(tabs[0][i]);
#pragma unroll
  for (int w = 1; w < 4; ++w) s += __uint_as_float(tabs[w][i]);
  return s;
}

__device__ __forceinline__ uint16_t bf16_lo_part(float v, uint16_t hi) {
  const float hf = bf16_bits_to_f32(hi);
  return fabsf(hf) <= 3.4028234663852886e38f ? f32_to_bf16_rne(v - hf) : (uint16_t)0;
}

__global__ __launch_bounds__(kMtThreads, 2) void gateup_mt_kernel(
    const uint16_t* __restrict__ x, uint32_t x_bytes, int k, int E, ExpertStore w, const int32_t* __restrict__ e2s,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, const uint8_t* __restrict__ run,
    uint16_t* __restrict__ hpl, int P) {
  constexpr int NF = kMtFrags, NG = NF / 2;
  __shared__ MtPlan pl;
  __shared__ uint32_t tabs[4][16 * NF * kMtW];
  __shared__ __attribute__((aligned(16))) uint8_t mtscr[4][NF * 2048];
  pl.build(offsets, E, run);
  const int H = w.H, I = w.I, NB = H / 32, tiles = I / (8 * NF), nch = H / 128;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, q16 = lane & 15, g = lane >> 4;
  const int cb = wid * nch / 4, ce = (wid + 1) * nch / 4;
  const uint32_t wrow = (uint32_t)H / 2u;
  const size_t mat = (size_t)I * wrow, smat = (size_t)I * NB, lo_plane = (size_t)P * I;
  const int units = tiles * pl.groups();
  uint32_t* tab = tabs[wid];
  // the gate/up epilogue of unit (b, mg, q): wavefront f < NG takes h columns
  // 8 NF q + 16f + q16 (gate fragment f, up fragment f + NG); accumulator v:
  // bucket row 16mg + 4g + v
  auto epilogue = [&](int mg, int q, int row0, int cnt, const f4v (&acc)[NF]) {
    __builtin_amdgcn_wave_barrier();
    mt_part_store<NF>(reinterpret_cast<float*>(tab), acc, lane);
    __syncthreads();
    if (wid < NG) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = kMtRows * mg + 4 * g + v;
        const float gv = mt_part_sum<NF>(tabs, wid, v, lane), uv = mt_part_sum<NF>(tabs, wid + NG, v, lane);
        if (row < cnt) {
          const float hv = swiglu_f32(gv, uv);
          const uint16_t hi = f32_to_bf16_rne(hv);
          const size_t o = (size_t)(row0 + row) * I + 8 * NF * q + 16 * wid + q16;
          hpl[o] = hi;
          hpl[lo_plane + o] = bf16_lo_part(hv, hi);
        }
      }
    }
    __syncthreads();  // the partials are read before the next unit's tables overwrite them
  };
  if ((nch + 3) / 4 <= kMtWin && nch / 4 >= 3) {  // every quarter one scale window of at least two sets
    auto make = [&](int u, GuUnit<NF>& U) {
      int b = 0, mg = 0, q = 0, slot = 0;
      for (; u < units; u += gridDim.x) {
        pl.locate(u, tiles, b, mg, q);
        const int expert = pl.bk.expert[b];
        slot = e2s ? e2s[expert] : expert;
        if (slot >= 0 && slot < w.num_slots) break;  // units of experts not stored: the down kernel writes zeros
      }
      U.u = u;
      U.live = u < units;
      const size_t sl = U.live ? (size_t)slot : 0;
      U.rg = make_rsrc(w.wg + sl * mat, (uint32_t)mat);
      U.ru = make_rsrc(w.wu + sl * mat, (uint32_t)mat);
      U.sg = make_rsrc(w.sg + sl * smat, (uint32_t)smat);
      U.su = make_rsrc(w.su + sl * smat, (uint32_t)smat);
      U.srow = (uint32_t)(8 * NF * q);
      U.boff = U.srow * wrow;
      const int row0 = U.live ? pl.bk.row0[b] : 0, cnt = U.live ? pl.bk.cnt[b] : 0;
      const int rr = kMtRows * mg + q16;
      U.pair = rr < cnt ? sorted_pair[row0 + rr] : -1;
      U.info[0] = mg, U.info[1] = q, U.info[2] = row0, U.info[3] = cnt;
    };
    auto va_of = [&](int pair) {
      return pair >= 0 ? (uint32_t)(pair / k) * (uint32_t)H * 2u + 64u * (uint32_t)g : kOob;
    };
    mt_gu_stream<NF>(blockIdx.x, gridDim.x, cb, ce, NB, 8u * wrow, make_rsrc(x, x_bytes), tab, mtscr[wid], make,
                     va_of, [&](const GuUnit<NF>& U, const f4v (&acc)[NF]) {
                       epilogue(U.info[0], U.info[1], U.info[2], U.info[3], acc);
                     });
    return;
  }
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    int b, mg, q;
    pl.locate(u, tiles, b, mg, q);
    const int expert = pl.bk.expert[b], row0 = pl.bk.row0[b], cnt = pl.bk.cnt[b];
    const int slot = e2s ? e2s[expert] : expert;
    if (slot < 0 || slot >= w.num_slots) continue;  // the down kernel writes zero rows
    const int rr = kMtRows * mg + q16;
    const int tok = rr < cnt ? sorted_pair[row0 + rr] / k : -1;
    MtSrc<1, NF> src;
    src.ra = make_rsrc(x, x_bytes);
    src.va = tok >= 0 ? (uint32_t)tok * (uint32_t)H * 2u + 64u * g : kOob;
    src.plane = 0;
    const rsrc_t gr = make_rsrc(w.wg + (size_t)slot * mat, (uint32_t)mat);
    const rsrc_t ur = make_rsrc(w.wu + (size_t)slot * mat, (uint32_t)mat);
#pragma unroll
    for (int f = 0; f < NF; ++f) {  // fragments 0 .. NG-1: gate rows; NG .. NF-1: the same up rows
      src.rb[f] = f < NG ? gr : ur;
      src.vb[f] = (uint32_t)(8 * NF * q + 16 * (f % NG) + (lane >> 3)) * wrow + 16u * (uint32_t)(lane & 7);
    }
    src.row8 = 8u * wrow;
    const rsrc_t sgr = make_rsrc(w.sg + (size_t)slot * smat, (uint32_t)smat);
    const rsrc_t sur = make_rsrc(w.su + (size_t)slot * smat, (uint32_t)smat);
    auto tables = [&](int cw0, MtTabGU<NF>& ts) {
      ts.t[0].issue(sgr, cw0, lane, [&](int r) { return (uint32_t)(8 * NF * q + r) * NB; });
      ts.t[1].issue(sur, cw0, lane, [&](int r) { return (uint32_t)(8 * NF * q + r) * NB; });
    };
    f4v acc[NF] = {};
    mt_k_loop_deep<MtTabGU<NF>>(src, acc, cb, ce, tab, mtscr[wid], tables);
    epilogue(mg, q, row0, cnt, acc);
  }
}

__global__ __launch_bounds__(kMtThreads, 2) void down_mt_kernel(
    const uint16_t* __restrict__ hpl, int P, int E, ExpertStore w, const int32_t* __restrict__ e2s,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair, const uint8_t* __restrict__ run,
    float* __restrict__ y) {
  constexpr int NF = kMtFrags;
  __shared__ MtPlan pl;
  __shared__ uint32_t tabs[4][16 * NF * kMtW];
  pl.build(offsets, E, run);
  const int H = w.H, I = w.I, NB = I / 32, tiles = H / (16 * NF), nch = I / 128;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, q16 = lane & 15, g = lane >> 4;
  const int cb = wid * nch / 4, ce = (wid + 1) * nch / 4;
  const uint32_t wrow = (uint32_t)I / 2u;
  const size_t mat = (size_t)H * wrow, smat = (size_t)H * NB;
  const int units = tiles * pl.groups();
  uint32_t* tab = tabs[wid];
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    int b, mg, q;
    pl.locate(u, tiles, b, mg, q);
    const int expert = pl.bk.expert[b], row0 = pl.bk.row0[b], cnt = pl.bk.cnt[b];
    const int slot = e2s ? e2s[expert] : expert;
    const int n0 = 16 * NF * q;
    if (slot < 0 || slot >= w.num_slots) {  // no stored expert: its rows are zero
      for (int r = kMtRows * mg + wid; r < min(cnt, kMtRows * (mg + 1)); r += 4)
        for (int c = lane; c < 16 * NF; c += 64) y[(size_t)sorted_pair[row0 + r] * H + n0 + c] = 0.f;
      continue;
    }
    const int rr = kMtRows * mg + q16;
    MtSrc<2, NF> src;
    src.ra = make_rsrc(hpl, (uint32_t)((size_t)P * I * 4));
    src.va = rr < cnt ? (uint32_t)(row0 + rr) * (uint32_t)I * 2u + 64u * g : kOob;
    src.plane = (uint32_t)((size_t)P * I * 2);
    const rsrc_t rc = make_rsrc(w.wd + (size_t)slot * mat, (uint32_t)mat);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      src.rb[f] = rc;
      src.vb[f] = (uint32_t)(n0 + 16 * f + q16) * wrow + 16u * (uint32_t)g;
    }
    src.row8 = 0;
    const rsrc_t sdr = make_rsrc(w.sd + (size_t)slot * smat, (uint32_t)smat);
    auto tables = [&](int cw0, MtTabDN<NF>& ts) {
      ts.t.issue(sdr, cw0, lane, [&](int r) { return (uint32_t)(n0 + r) * NB; });
    };
    f4v acc[NF] = {};
    mt_k_loop<MtTabDN<NF>>(src, acc, cb, ce, tab, tables);
    __builtin_amdgcn_wave_barrier();
    mt_part_store<NF>(reinterpret_cast<float*>(tab), acc, lane);
    __syncthreads();
    // fragment f (wavefront f % 4): output columns n0 + 16f + q16; accumulator v: bucket row 16mg + 4g + v
    for (int f = wid; f < NF; f += 4) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = kMtRows * mg + 4 * g + v;
        const float yv = mt_part_sum<NF>(tabs, f, v, lane);
        if (row < cnt) y[(size_t)sorted_pair[row0 + row] * H + n0 + 16 * f + q16] = yv;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// The batch-invariant decode layer of one token in one call: route + gate/up,
// then down, then the fixed-order combine.  Every output is computed by the
// arithmetic of gateup_mt_kernel and down_mt_kernel (the same K quarters,
// chunk order and MFMA sequence, the same partial-sum order), so the token's
// rows are bit-identical to its rows in a batch; the routing runs in every
// workgroup of the first kernel (as the fast one-token layer does), which
// saves the route and permute launches and the plan of the buckets.
// ---------------------------------------------------------------------------

struct InvRoute {
  int expert[kMaxTopK];  // bucket order: ascending expert id
  int slot[kMaxTopK];    // storage slot of bucket b's expert (-1: none)
  int pair[kMaxTopK];    // routing slot j of bucket b (its y_pair row)
};

// Wavefront 0 routes the token (route_token) and ranks the k picks by expert
// id, the bucket order of moe_permute; workgroup 0 publishes the routing.
// Ends on a barrier.
template <int NPL>
__device__ void inv_route(const float* __restrict__ logits, int E, int k, const int32_t* __restrict__ e2s,
                          int num_slots, InvRoute& r, InvRoute* __restrict__ pub, int32_t* __restrict__ topk_ids,
                          float* __restrict__ topk_w) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const RoutePick pick = route_token<NPL>(logits, E, k, e2s, lane);
    int rank = 0;
    for (int i = 0; i < k; ++i) {
      const int ei = __builtin_amdgcn_readlane(pick.expert, i);
      rank += (ei < pick.expert || (ei == pick.expert && i < lane)) ? 1 : 0;
    }
    if (lane < k) {
      int sl = e2s ? e2s[pick.expert] : pick.expert;
      if (sl >= num_slots) sl = -1;
      r.expert[rank] = pick.expert;
      r.slot[rank] = sl;
      r.pair[rank] = lane;
      if (blockIdx.x == 0) {
        topk_ids[lane] = pick.expert;
        topk_w[lane] = pick.weight;
        pub->expert[rank] = pick.expert;
        pub->slot[rank] = sl;
        pub->pair[rank] = lane;
      }
    }
  }
  __syncthreads();
}

// gateup_mt_kernel for the one routed token: unit u = (bucket u / tiles,
// column tile u % tiles); the token is row 0 of the unit's 16-row group.
template <int NPL>
__global__ __launch_bounds__(kMtThreads, 2) void inv_gateup_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int E, int k, const int32_t* __restrict__ e2s,
    ExpertStore w, InvRoute* __restrict__ pub, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    uint16_t* __restrict__ hpl) {
  constexpr int NF = kMtFrags, NG = NF / 2;
  __shared__ InvRoute rt;
  __shared__ uint32_t tabs[4][16 * NF * kMtW];
  __shared__ __attribute__((aligned(16))) uint8_t mtscr[4][NF * 2048];
  inv_route<NPL>(logits, E, k, e2s, w.num_slots, rt, pub, topk_ids, topk_w);
  const int H = w.H, I = w.I, NB = H / 32, tiles = I / (8 * NF), nch = H / 128;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, q16 = lane & 15, g = lane >> 4;
  const int cb = wid * nch / 4, ce = (wid + 1) * nch / 4;
  const uint32_t wrow = (uint32_t)H / 2u;
  const size_t mat = (size_t)I * wrow, smat = (size_t)I * NB, lo_plane = (size_t)k * I;
  const int units = k * tiles;
  uint32_t* tab = tabs[wid];
  // wavefront f < NG: h columns 8 NF q + 16f + q16; the token is accumulator 0 of lanes 0-15
  auto epilogue = [&](int b, int q, const f4v (&acc)[NF]) {
    __builtin_amdgcn_wave_barrier();
    mt_part_store<NF>(reinterpret_cast<float*>(tab), acc, lane);
    __syncthreads();
    if (wid < NG && g == 0) {
      const float gv = mt_part_sum<NF>(tabs, wid, 0, lane), uv = mt_part_sum<NF>(tabs, wid + NG, 0, lane);
      const float hv = swiglu_f32(gv, uv);
      const uint16_t hi = f32_to_bf16_rne(hv);
      const size_t o = (size_t)b * I + 8 * NF * q + 16 * wid + q16;
      hpl[o] = hi;
      hpl[lo_plane + o] = bf16_lo_part(hv, hi);
    }
    __syncthreads();  // the partials are read before the next unit's tables overwrite them
  };
  if ((nch + 3) / 4 <= kMtWin && nch / 4 >= 3) {  // every quarter one scale window of at least two sets
    auto make = [&](int u, GuUnit<NF>& U) {
      int slot = -1;
      for (; u < units; u += gridDim.x) {
        slot = rt.slot[u / tiles];
        if (slot >= 0) break;  // buckets of experts not stored: the down kernel writes zero rows
      }
      U.u = u;
      U.live = u < units;
      const int b = U.live ? u / tiles : 0, q = U.live ? u - b * tiles : 0;
      const size_t sl = U.live ? (size_t)slot : 0;
      U.rg = make_rsrc(w.wg + sl * mat, (uint32_t)mat);
      U.ru = make_rsrc(w.wu + sl * mat, (uint32_t)mat);
      U.sg = make_rsrc(w.sg + sl * smat, (uint32_t)smat);
      U.su = make_rsrc(w.su + sl * smat, (uint32_t)smat);
      U.srow = (uint32_t)(8 * NF * q);
      U.boff = U.srow * wrow;
      U.pair = 0;
      U.info[0] = b, U.info[1] = q;
    };
    auto va_of = [&](int) { return q16 == 0 ? 64u * (uint32_t)g : kOob; };
    mt_gu_stream<NF>(blockIdx.x, gridDim.x, cb, ce, NB, 8u * wrow, make_rsrc(x, (uint32_t)H * 2u), tab, mtscr[wid],
                     make, va_of, [&](const GuUnit<NF>& U, const f4v (&acc)[NF]) { epilogue(U.info[0], U.info[1], acc); });
    return;
  }
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int b = u / tiles, q = u - b * tiles;
    const int slot = rt.slot[b];
    if (slot < 0) continue;  // the down kernel writes zero rows
    MtSrc<1, NF> src;
    src.ra = make_rsrc(x, (uint32_t)H * 2u);
    src.va = q16 == 0 ? 64u * g : kOob;
    src.plane = 0;
    const rsrc_t gr = make_rsrc(w.wg + (size_t)slot * mat, (uint32_t)mat);
    const rsrc_t ur = make_rsrc(w.wu + (size_t)slot * mat, (uint32_t)mat);
#pragma unroll
    for (int f = 0; f < NF; ++f) {  // fragments 0 .. NG-1: gate rows; NG .. NF-1: the same up rows
      src.rb[f] = f < NG ? gr : ur;
      src.vb[f] = (uint32_t)(8 * NF * q + 16 * (f % NG) + (lane >> 3)) * wrow + 16u * (uint32_t)(lane & 7);
    }
    src.row8 = 8u * wrow;
    const rsrc_t sgr = make_rsrc(w.sg + (size_t)slot * smat, (uint32_t)smat);
    const rsrc_t sur = make_rsrc(w.su + (size_t)slot * smat, (uint32_t)smat);
    auto tables = [&](int cw0, MtTabGU<NF>& ts) {
      ts.t[0].issue(sgr, cw0, lane, [&](int r) { return (uint32_t)(8 * NF * q + r) * NB; });
      ts.t[1].issue(sur, cw0, lane, [&](int r) { return (uint32_t)(8 * NF * q + r) * NB; });
    };
    f4v acc[NF] = {};
    mt_k_loop_deep<MtTabGU<NF>>(src, acc, cb, ce, tab, mtscr[wid], tables);
    epilogue(b, q, acc);
  }
}

// down_mt_kernel for the one routed token: unit u = (bucket u / tiles, 16 NF
// output columns u % tiles); y_pair row = the bucket's routing slot.
__global__ __launch_bounds__(kMtThreads, 2) void inv_down_kernel(int k, ExpertStore w,
                                                                 const InvRoute* __restrict__ pub,
                                                                 const uint16_t* __restrict__ hpl,
                                                                 float* __restrict__ y) {
  constexpr int NF = kMtFrags;
  __shared__ InvRoute rt;
  __shared__ uint32_t tabs[4][16 * NF * kMtW];
  if (threadIdx.x < kMaxTopK) {
    rt.expert[threadIdx.x] = pub->expert[threadIdx.x];
    rt.slot[threadIdx.x] = pub->slot[threadIdx.x];
    rt.pair[threadIdx.x] = pub->pair[threadIdx.x];
  }
  __syncthreads();
  const int H = w.H, I = w.I, NB = I / 32, tiles = H / (16 * NF), nch = I / 128;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, q16 = lane & 15, g = lane >> 4;
  const int cb = wid * nch / 4, ce = (wid + 1) * nch / 4;
  const uint32_t wrow = (uint32_t)I / 2u;
  const size_t mat = (size_t)H * wrow, smat = (size_t)H * NB;
  const int units = k * tiles;
  uint32_t* tab = tabs[wid];
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int b = u / tiles, q = u - b * tiles;
    const int slot = rt.slot[b], n0 = 16 * NF * q;
    float* yrow = y + (size_t)rt.pair[b] * H;
    if (slot < 0) {  // no stored expert: its row is zero
      if (wid == 0)
        for (int c = lane; c < 16 * NF; c += 64) yrow[n0 + c] = 0.f;
      continue;
    }
    MtSrc<2, NF> src;
    src.ra = make_rsrc(hpl, (uint32_t)((size_t)k * I * 4));
    src.va = q16 == 0 ? (uint32_t)b * (uint32_t)I * 2u + 64u * g : kOob;
    src.plane = (uint32_t)((size_t)k * I * 2);
    const rsrc_t rc = make_rsrc(w.wd + (size_t)slot * mat, (uint32_t)mat);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      src.rb[f] = rc;
      src.vb[f] = (uint32_t)(n0 + 16 * f + q16) * wrow + 16u * (uint32_t)g;
    }
    src.row8 = 0;
    const rsrc_t sdr = make_rsrc(w.sd + (size_t)slot * smat, (uint32_t)smat);
    auto tables = [&](int cw0, MtTabDN<NF>& ts) {
      ts.t.issue(sdr, cw0, lane, [&](int r) { return (uint32_t)(n0 + r) * NB; });
    };
    f4v acc[NF] = {};
    mt_k_loop<MtTabDN<NF>>(src, acc, cb, ce, tab, tables);
    __builtin_amdgcn_wave_barrier();
    mt_part_store<NF>(reinterpret_cast<float*>(tab), acc, lane);
    __syncthreads();
    // fragment f (wavefront f % 4): output columns n0 + 16f + q16; the token is accumulator 0 of lanes 0-15
    if (g == 0)
      for (int f = wid; f < NF; f += 4) yrow[n0 + 16 * f + q16] = mt_part_sum<NF>(tabs, f, 0, lane);
    __syncthreads();
  }
}

}  // namespace

size_t invariant_layer_workspace_bytes(int k, int H, int I) {
  return 256 + (((size_t)k * I * 4 + 255) & ~(size_t)255) + (size_t)k * H * 4;
}

hipError_t launch_invariant_layer(const float* logits, const uint16_t* x, int E, int k, const int32_t* e2s,
                                  const ExpertStore& w, const uint16_t* residual, bool bf16_out, void* out,
                                  int32_t* topk_ids, float* topk_w, void* ws, hipStream_t s) {
  InvRoute* pub = reinterpret_cast<InvRoute*>(ws);
  uint16_t* hpl = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(ws) + 256);
  float* y = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + 256 +
                                      (((size_t)k * w.I * 4 + 255) & ~(size_t)255));
  const int npl = (E + 63) / 64;
  const dim3 g1(min(k * (w.I / (8 * kMtFrags)), kMtGridGU)), b1(kMtThreads);
#define MOE_INV_GU(NP) \
  hipLaunchKernelGGL(inv_gateup_kernel<NP>, g1, b1, 0, s, logits, x, E, k, e2s, w, pub, topk_ids, topk_w, hpl)
  if (npl <= 1) MOE_INV_GU(1);
  else if (npl <= 2) MOE_INV_GU(2);
  else if (npl <= 4) MOE_INV_GU(4);
  else if (npl <= 8) MOE_INV_GU(8);
  else MOE_INV_GU(16);
#undef MOE_INV_GU
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(inv_down_kernel, dim3(min(k * (w.H / (16 * kMtFrags)), kMtGridDN)), dim3(kMtThreads), 0, s, k,
                     w, pub, hpl, y);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(y, topk_w, 1, k, w.H, residual, bf16_out, out, s);
}

hipError_t launch_decode_mt(const uint16_t* x, int T, int k, int E, const ExpertStore& w, const int32_t* e2s,
                            const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws, int phase,
                            hipStream_t s, const uint8_t* run) {
  const int P = T * k;
  uint16_t* hpl = reinterpret_cast<uint16_t*>(ws);
  if (phase != 2) {
    hipLaunchKernelGGL(gateup_mt_kernel, dim3(kMtGridGU), dim3(kMtThreads), 0, s, x,
                       (uint32_t)((size_t)T * w.H * 2), k, E, w, e2s, offsets, sorted_pair, run, hpl, P);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || phase == 1) return err;
  }
  hipLaunchKernelGGL(down_mt_kernel, dim3(kMtGridDN), dim3(kMtThreads), 0, s, hpl, P, E, w, e2s, offsets,
                     sorted_pair, run, y_pair);
  return hipGetLastError();
}

}  // namespace moe
