// Decode FFN over experts in the 3-bit per-row codebook format (gfx950).
//
// The DGX Spark page ("The numbers") stores its routable experts as 3-bit
// indices into a small codebook per output row, repacked from the model's
// FP4 experts.  Format read here: every output row has 8 bf16 codebook entries (16 bytes, one
// uint4); each weight is a 3-bit index, 8 indices per 3 bytes (bits 3i..3i+2
// of a little-endian 24-bit word).  A row of K weights is 3K/8 bytes, 0.71x
// the e2m1 codes plus UE8M0 scales of the same row.
//
// Arithmetic is the decode reference's ("Fast single-box DeepSeek v4.1 Flash
// runtime", "Conventions"): x stays bf16, so W.x uses exact bf16 products
// summed in fp32 (v_dot2_f32_bf16), and h stays fp32 for the down projection
// (fp32 FMAs).  Two indices are decoded at once: for every row of a unit the
// wavefront writes a 64-entry table of codebook pairs into its own LDS area
// (entry a + 8b = entry a in the low half, entry b in the high half; lane l
// writes entry l), and each pair of weights is one ds_read_b32 of it.
//
// Work: a gate/up unit is (bucket, one row of W_gate and the same row of
// W_up), a down unit (bucket, four output rows).  Each wavefront takes one
// contiguous range of units, keeps the x row (gate/up) or h row (down) of its
// current bucket row in registers while consecutive units share it, and
// loads the next unit's index words and codebooks while it computes the
// current one.  Lane l takes the 32-weight groups l, l+64, ... of a row; in
// the down kernel the groups left over past the last multiple of 64 are
// dealt out as (row, group) items over all lanes instead.  Every bucket row
// (token) of a unit reuses the unit's index words and codebooks, decoding
// them again.
#include "common.cuh"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCbThreads = 256;
constexpr int kCbGridGU = 768;  // three workgroups per CU: the gate/up kernel fits three wavefronts per SIMD
constexpr int kCbGridDN = 512;  // the down kernel fits two
constexpr int kCbDnRows = 4;    // output rows per down unit
constexpr int kCbGU = 3;  // 32-weight groups per lane of a gate/up row: hidden <= 64*32*3 = 6144
constexpr int kCbDN = 2;  // ... of a down row: inter <= 4096

// Entry a + 8b of a row's pair table (a = l & 7, b = l >> 3): codebook
// entries a and b as one bf16x2 word, a in the low half.  ca and cb are the
// codebook words that hold entries a and b (entry 2i is the low half of word i).
__device__ __forceinline__ uint32_t cb3_table_entry(int l, uint32_t ca, uint32_t cb) {
  const int a = l & 7, b = l >> 3;
  return ((ca >> (16 * (a & 1))) & 0xFFFFu) | (((cb >> (16 * (b & 1))) & 0xFFFFu) << 16);
}

typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// LDS byte address of a 256-byte-aligned pair table.
__device__ __forceinline__ uint32_t lds_addr(const uint32_t* tab) { return (uint32_t)(size_t)(lds_u32*)tab; }

// The 16 bf16x2 weight words of one 32-weight group from its 12 index bytes
// (w.x, w.y, w.z) and the row's pair table at LDS address base (256-byte
// aligned): word 4s + j holds weights 8s + 2j and 8s + 2j + 1, whose 6-bit
// pair index is the table entry.  Each 24-bit index word is taken shifted
// left by two, so entry j's byte offset is one shift and one AND-OR with the
// base away.
__device__ __forceinline__ void cb3_group(uint3 w, uint32_t base, uint32_t (&out)[16]) {
  // an empty statement that claims to change the index words: the sixteen
  // addresses are formed here, at their use, instead of being hoisted out of
  // the caller's loop over bucket rows and kept live in registers
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z));
  const uint32_t g[4] = {w.x << 2, __builtin_amdgcn_alignbit(w.y, w.x, 22), __builtin_amdgcn_alignbit(w.z, w.y, 14),
                         w.z >> 6};  // bits past 25 are never read
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * s + j] = *(lds_u32*)(size_t)(((g[s] >> (6 * j)) & 0xFCu) | base);
}

__device__ __forceinline__ uint3 bload12(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
  return make_uint3(v[0], v[1], v[2]);
}

// One stored row's index words (lane l: groups l, l+64, ...) and codebook.
// Every load is issued unconditionally: a row that is absent (a unit past the
// end, an expert with no stored slot) has an empty range and reads zeros, and
// groups past the row's end read zeros, so the compiler counts the loads in
// flight exactly and a wavefront can compute one unit while the next unit's
// rows are on the way.
template <int NGL>
__device__ __forceinline__ void cb3_row_load(const uint8_t* q, const uint16_t* cb, size_t row, bool ok,
                                             uint32_t qrow, int NG, int lane, uint3 (&qv)[NGL], uint2& cv) {
  const rsrc_t rq = make_rsrc(q + (ok ? row * qrow : 0), ok ? qrow : 0u);
  const rsrc_t rc = make_rsrc(cb + (ok ? row * 8 : 0), ok ? 16u : 0u);
  // the two codebook words this lane's table entry needs
  cv = make_uint2(bload4(rc, 4u * (uint32_t)((lane & 7) >> 1)), bload4(rc, 4u * (uint32_t)(lane >> 4)));
#pragma unroll
  for (int gi = 0; gi < NGL; ++gi) {
    const int G = lane + 64 * gi;
    qv[gi] = bload12(rq, G < NG ? 12u * (uint32_t)G : kOob);
  }
}

// A unit's place: bucket b and the stored slot of its expert (ok = false
// for a unit past the end or an expert with no stored slot).
struct Cb3Unit {
  int b, rest, slot;
  bool live, ok;
};

__device__ __forceinline__ Cb3Unit cb3_unit(int unit, int units, int per_bucket, const Buckets& bk,
                                            const int32_t* __restrict__ e2s, int num_slots) {
  Cb3Unit u;
  u.live = unit < units;
  u.b = u.live ? unit / per_bucket : 0;
  u.rest = u.live ? unit - u.b * per_bucket : 0;
  // wave-uniform, so the e2s lookup is a scalar load and no vector-load wait
  // lands between a unit's x loads and the next unit's prefetch
  const int expert = __builtin_amdgcn_readfirstlane(bk.expert[u.b]);
  u.slot = u.live ? (e2s ? e2s[expert] : expert) : -1;
  u.ok = u.slot >= 0 && u.slot < num_slots;
  return u;
}

__global__ __launch_bounds__(kCbThreads, 3) void cb3_gateup_kernel(const uint16_t* __restrict__ x, int k, int E,
                                                                   Cb3Store w, const int32_t* __restrict__ e2s,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ sorted_pair,
                                                                   float* __restrict__ h) {
  __shared__ Buckets bk;
  __shared__ __attribute__((aligned(256))) uint32_t tabs[4][2][64];  // per wavefront: the pair tables of its unit's gate and up rows
  build_buckets(offsets, E, bk, nullptr);
  const int lane = threadIdx.x & 63;
  uint32_t (*tab)[64] = tabs[threadIdx.x >> 6];
  const int H = w.H, I = w.I, NG = H / 32;
  const uint32_t qrow = (uint32_t)H * 3 / 8;
  // each wavefront takes one contiguous range of units, so consecutive units
  // mostly share the bucket (and, for one token, the x row)
  const int units = bk.n * I, nw = gridDim.x * 4, per = (units + nw - 1) / nw;
  int unit = (blockIdx.x * 4 + (threadIdx.x >> 6)) * per;
  const int uend = min(units, unit + per);
  // row n of gate (m = 0) and up (m = 1): index words and codebooks
  uint3 q[2][kCbGU], nq[2][kCbGU];
  uint2 cb[2], ncb[2];
  Cb3Unit u = cb3_unit(unit, units, I, bk, e2s, w.num_slots);
  cb3_row_load(w.qg, w.cg, (size_t)u.slot * I + u.rest, u.ok, qrow, NG, lane, q[0], cb[0]);
  cb3_row_load(w.qu, w.cu, (size_t)u.slot * I + u.rest, u.ok, qrow, NG, lane, q[1], cb[1]);
  // the x row of a token: lane l's groups, 64 bytes each
  auto load_x = [&](int token, uint4_t (&xv)[kCbGU][4]) {
    const rsrc_t rx = make_rsrc(x + (size_t)token * H, 2u * (uint32_t)H);
#pragma unroll
    for (int gi = 0; gi < kCbGU; ++gi) {
      const int G = lane + 64 * gi;
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[gi][c] = bload16(rx, G < NG ? 64u * (uint32_t)G + 16u * c : kOob);
    }
  };
  uint4_t xv[kCbGU][4];
  int xtok = -1;  // the token whose x row is in xv
  for (; unit < uend; ++unit) {
    const int n = u.rest, row0 = bk.row0[u.b], cnt = bk.cnt[u.b];
    const bool ok = u.ok;
    // the previous unit's table reads are done: a wavefront's LDS accesses complete in order
#pragma unroll
    for (int m = 0; m < 2; ++m) tab[m][lane] = cb3_table_entry(lane, cb[m].x, cb[m].y);
    __builtin_amdgcn_wave_barrier();
    const Cb3Unit un = cb3_unit(unit + 1 < uend ? unit + 1 : units, units, I, bk, e2s, w.num_slots);
    if (const int t0 = sorted_pair[row0] / k; t0 != xtok) {
      load_x(t0, xv);
      xtok = t0;
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next unit's rows, in flight behind this unit's first x row
    cb3_row_load(w.qg, w.cg, (size_t)un.slot * I + un.rest, un.ok, qrow, NG, lane, nq[0], ncb[0]);
    cb3_row_load(w.qu, w.cu, (size_t)un.slot * I + un.rest, un.ok, qrow, NG, lane, nq[1], ncb[1]);
    __builtin_amdgcn_sched_barrier(0);
    {  // a unit with no stored slot reads zeros and stores nothing: the down kernel writes zero rows
      for (int r = 0; r < cnt; ++r) {
        if (const int t = sorted_pair[row0 + r] / k; t != xtok) {
          load_x(t, xv);
          xtok = t;
        }
        float acc[2] = {0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < kCbGU; ++gi) {
          const int G = lane + 64 * gi;
          if (G >= NG) break;
          const uint32_t xw[16] = {xv[gi][0][0], xv[gi][0][1], xv[gi][0][2], xv[gi][0][3],
                                   xv[gi][1][0], xv[gi][1][1], xv[gi][1][2], xv[gi][1][3],
                                   xv[gi][2][0], xv[gi][2][1], xv[gi][2][2], xv[gi][2][3],
                                   xv[gi][3][0], xv[gi][3][1], xv[gi][3][2], xv[gi][3][3]};
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            uint32_t wv[16];
            cb3_group(q[m][gi], lds_addr(tab[m]), wv);
            float a = acc[m];
#pragma unroll
            for (int t = 0; t < 16; ++t)
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv[t]),
                                                  __builtin_bit_cast(bf16x2_t, xw[t]), a, false);
            acc[m] = a;
            __builtin_amdgcn_sched_barrier(0);  // one row's table reads live at a time
          }
        }
        // reduce (gate, up) over the wavefront: after the swap lanes 0-31 carry
        // gate partials and 32-63 up partials; the 16-lane sums of rows 0 + 1 and
        // 2 + 3 are added in that order
        const float a = sum16(tswap32(acc[0], acc[1]));
        const float gs = lane_value(a, 0) + lane_value(a, 16), us = lane_value(a, 32) + lane_value(a, 48);
        if (ok && lane == 0) h[(size_t)(row0 + r) * I + n] = swiglu_f32(gs, us);
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      cb[m] = ncb[m];
#pragma unroll
      for (int gi = 0; gi < kCbGU; ++gi) q[m][gi] = nq[m][gi];
    }
    u = un;
  }
}

template <int R>
__global__ __launch_bounds__(kCbThreads, 2) void cb3_down_kernel(int k, int E, Cb3Store w,
                                                                 const int32_t* __restrict__ e2s,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ sorted_pair,
                                                                 const float* __restrict__ h, float* __restrict__ y) {
  __shared__ Buckets bk;
  __shared__ __attribute__((aligned(256))) uint32_t tabs[4][R][64];  // per wavefront: the pair tables of its unit's R rows
  build_buckets(offsets, E, bk, nullptr);
  const int lane = threadIdx.x & 63;
  uint32_t (*tab)[64] = tabs[threadIdx.x >> 6];
  const int H = w.H, I = w.I, NG = I / 32;
  const uint32_t qrow = (uint32_t)I * 3 / 8;
  // groups 0 .. 64*FULL-1 of a row: lane l takes groups l, l+64, ... of every
  // row of the unit; the NT groups left over are R*NT (row, group) items dealt
  // out over the lanes, so no pass runs with most lanes idle
  const int FULL = NG / 64, NGM = 64 * FULL, NT = NG - NGM, NTI = R * NT;
  // each wavefront takes one contiguous range of units, so consecutive units
  // mostly share the bucket and its h rows
  const int units = bk.n * (H / R), nw = gridDim.x * 4, per = (units + nw - 1) / nw;
  int unit = (blockIdx.x * 4 + (threadIdx.x >> 6)) * per;
  const int uend = min(units, unit + per);
  uint3 q[R][kCbDN], nq[R][kCbDN];
  uint2 cb[R], ncb[R];
  Cb3Unit u = cb3_unit(unit, units, H / R, bk, e2s, w.num_slots);
#pragma unroll
  for (int i = 0; i < R; ++i)
    cb3_row_load(w.qd, w.cd, (size_t)u.slot * H + R * u.rest + i, u.ok, qrow, NGM, lane, q[i], cb[i]);
  static_assert(R == 2 || R == 4, "two or four rows per unit");
  // the h row of a bucket row: lane l's groups, 128 bytes each
  auto load_h = [&](int brow, float4_t (&hv)[kCbDN][8]) {
    const rsrc_t rh = make_rsrc(h + (size_t)brow * I, 4u * (uint32_t)I);
#pragma unroll
    for (int gi = 0; gi < kCbDN; ++gi) {
      const int G = lane + 64 * gi;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4_t t = bload16(rh, G < NGM ? 128u * (uint32_t)G + 16u * c : kOob);
        hv[gi][c] = float4_t{__uint_as_float(t[0]), __uint_as_float(t[1]), __uint_as_float(t[2]),
                             __uint_as_float(t[3])};
      }
    }
  };
  float4_t hv[kCbDN][8];
  int hrow = -1;  // the bucket row whose h is in hv
  for (; unit < uend; ++unit) {
    const int m0 = R * u.rest, row0 = bk.row0[u.b], cnt = bk.cnt[u.b];
    const bool ok = u.ok;
#pragma unroll
    for (int i = 0; i < R; ++i) tab[i][lane] = cb3_table_entry(lane, cb[i].x, cb[i].y);
    __builtin_amdgcn_wave_barrier();
    const Cb3Unit un = cb3_unit(unit + 1 < uend ? unit + 1 : units, units, H / R, bk, e2s, w.num_slots);
    if (row0 != hrow) {
      load_h(row0, hv);
      hrow = row0;
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next unit's rows, in flight behind this unit's first h row
#pragma unroll
    for (int i = 0; i < R; ++i)
      cb3_row_load(w.qd, w.cd, (size_t)un.slot * H + R * un.rest + i, un.ok, qrow, NGM, lane, nq[i], ncb[i]);
    __builtin_amdgcn_sched_barrier(0);
    {  // a unit with no stored expert reads zero weights: its rows are written as zeros
      for (int r = 0; r < cnt; ++r) {
        if (row0 + r != hrow) {
          load_h(row0 + r, hv);
          hrow = row0 + r;
        }
        float v[R] = {};
        const uint32_t tb = lds_addr(tab[0]);  // row i's table at tb + 256 i
#pragma unroll
        for (int gi = 0; gi < kCbDN; ++gi) {
          if (gi >= FULL) break;
#pragma unroll
          for (int i = 0; i < R; ++i) {
            uint32_t wv[16];
            cb3_group(q[i][gi], tb + 256u * i, wv);
            float a = v[i];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
              const float4_t& hc = hv[gi][t >> 1];
              a = fmaf(bf16_bits_to_f32(wv[t] & 0xFFFFu), (t & 1) ? hc.z : hc.x, a);
              a = fmaf(bf16_bits_to_f32(wv[t] >> 16), (t & 1) ? hc.w : hc.y, a);
            }
            v[i] = a;
            __builtin_amdgcn_sched_barrier(0);  // one row's table reads live at a time
          }
        }
        // the tail items: item = lane + 64p is row item / NT, group NGM + item % NT
        for (int p0 = 0; p0 < NTI; p0 += 64) {
          const int item = p0 + lane;
          const bool on = item < NTI;
          const int i = on ? item / NT : 0, G = NGM + (on ? item - i * NT : 0);
          const rsrc_t rq = make_rsrc(w.qd + (ok ? ((size_t)u.slot * H + m0) * qrow : 0), ok ? R * qrow : 0u);
          const rsrc_t rh = make_rsrc(h + (size_t)(row0 + r) * I, 4u * (uint32_t)I);
          const uint3 qt = bload12(rq, on ? (uint32_t)i * qrow + 12u * (uint32_t)G : kOob);
          float4_t ht[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint4_t t = bload16(rh, on ? 128u * (uint32_t)G + 16u * c : kOob);
            ht[c] = float4_t{__uint_as_float(t[0]), __uint_as_float(t[1]), __uint_as_float(t[2]), __uint_as_float(t[3])};
          }
          uint32_t wv[16];
          cb3_group(qt, tb + 256u * (uint32_t)i, wv);
          float a = 0.f;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const float4_t& hc = ht[t >> 1];
            a = fmaf(bf16_bits_to_f32(wv[t] & 0xFFFFu), (t & 1) ? hc.z : hc.x, a);
            a = fmaf(bf16_bits_to_f32(wv[t] >> 16), (t & 1) ? hc.w : hc.y, a);
          }
#pragma unroll
          for (int ii = 0; ii < R; ++ii) v[ii] += (on && i == ii) ? a : 0.f;
        }
        if constexpr (R == 4) {  // 4 row partials -> lane 16i holds the sum of row i
          const float a0 = tswap32(v[0], v[2]), a1 = tswap32(v[1], v[3]);
          const float c = sum16(tswap16(a0, a1));
          if ((lane & 15) == 0) y[(size_t)sorted_pair[row0 + r] * H + m0 + (lane >> 4)] = ok ? c : 0.f;
        } else {  // 2 row partials -> the 16-lane sums of lanes 0-31 (row 0) and 32-63 (row 1)
          const float c = sum16(tswap32(v[0], v[1]));
          const float r0 = lane_value(c, 0) + lane_value(c, 16), r1 = lane_value(c, 32) + lane_value(c, 48);
          if (lane < 2) y[(size_t)sorted_pair[row0 + r] * H + m0 + lane] = ok ? (lane == 0 ? r0 : r1) : 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      cb[i] = ncb[i];
#pragma unroll
      for (int gi = 0; gi < kCbDN; ++gi) q[i][gi] = nq[i][gi];
    }
    u = un;
  }
}

}  // namespace

bool cb3_decode_supported(int H, int I) {
  return H % 256 == 0 && H / 32 <= 64 * kCbGU && I % 128 == 0 && I / 32 <= 64 * kCbDN;
}

hipError_t launch_decode_cb3(const uint16_t* x, int T, int k, int E, const Cb3Store& w, const int32_t* e2s,
                             const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws,
                             hipStream_t s) {
  (void)T;
  float* h = reinterpret_cast<float*>(ws);
  hipLaunchKernelGGL(cb3_gateup_kernel, dim3(kCbGridGU), dim3(kCbThreads), 0, s, x, k, E, w, e2s, offsets,
                     sorted_pair, h);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(cb3_down_kernel<kCbDnRows>, dim3(kCbGridDN), dim3(kCbThreads), 0, s, k, E, w, e2s, offsets, sorted_pair, h,
                     y_pair);
  return hipGetLastError();
}

}  // namespace moe
