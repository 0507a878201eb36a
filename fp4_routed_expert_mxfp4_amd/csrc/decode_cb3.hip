// Decode FFN over experts in the 3-bit per-row codebook format (gfx950).
//
// The DGX Spark page ("The numbers") keeps its routable experts "in a 3-bit
// per-row codebook packed from the checkpoint's own FP4 experts".  Format
// read here: every output row has 8 bf16 codebook entries (16 bytes, one
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
// Lane l of a wavefront takes the 32-weight groups l, l+64, ... of a row; a
// gate/up unit is (bucket, one row of W_gate and the same row of W_up), a
// down unit (bucket, four output rows).  Every bucket row (token) of a unit
// reuses the unit's index words and codebooks, decoding them again.
#include "common.cuh"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCbThreads = 256;
constexpr int kCbGridGU = 768;  // three workgroups per CU: the gate/up kernel fits three wavefronts per SIMD
constexpr int kCbGridDN = 512;  // the down kernel (four rows per unit) fits two
constexpr int kCbGU = 3;  // 32-weight groups per lane of a gate/up row: hidden <= 64*32*3 = 6144
constexpr int kCbDN = 2;  // ... of a down row: inter <= 4096

// Entry a + 8b of a row's pair table: codebook entries a and b (entry 2i in
// the low half of word i of cb) as one bf16x2 word, a in the low half.
__device__ __forceinline__ uint32_t cb3_table_entry(int l, const uint4& cb) {
  const uint32_t w[4] = {cb.x, cb.y, cb.z, cb.w};
  const int a = l & 7, b = l >> 3;
  const uint32_t ea = (w[a >> 1] >> (16 * (a & 1))) & 0xFFFFu;
  const uint32_t eb = (w[b >> 1] >> (16 * (b & 1))) & 0xFFFFu;
  return ea | (eb << 16);
}

// The 16 bf16x2 weight words of one 32-weight group from its 12 index bytes
// (w.x, w.y, w.z) and the row's pair table: word 4s + j holds weights 8s + 2j
// and 8s + 2j + 1 (the 6-bit pair index is the table entry).
__device__ __forceinline__ void cb3_group(const uint3& w, const uint32_t* tab, uint32_t (&out)[16]) {
  const uint32_t g[4] = {w.x & 0xFFFFFFu, (w.x >> 24) | ((w.y & 0xFFFFu) << 8), (w.y >> 16) | ((w.z & 0xFFu) << 16),
                         w.z >> 8};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * s + j] = tab[(g[s] >> (6 * j)) & 63u];
}

__device__ __forceinline__ uint3 ld12(const uint8_t* p) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  return make_uint3(q[0], q[1], q[2]);
}

__device__ __forceinline__ uint4 ld_cb(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__global__ __launch_bounds__(kCbThreads, 3) void cb3_gateup_kernel(const uint16_t* __restrict__ x, int k, int E,
                                                                   Cb3Store w, const int32_t* __restrict__ e2s,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ sorted_pair,
                                                                   float* __restrict__ h) {
  __shared__ Buckets bk;
  __shared__ uint32_t tabs[4][2][64];  // per wavefront: the pair tables of its unit's gate and up rows
  build_buckets(offsets, E, bk, nullptr);
  const int lane = threadIdx.x & 63;
  uint32_t (*tab)[64] = tabs[threadIdx.x >> 6];
  const int H = w.H, I = w.I, NG = H / 32;
  const size_t qrow = (size_t)H * 3 / 8;
  const int units = bk.n * I;
  for (int unit = blockIdx.x * 4 + (threadIdx.x >> 6); unit < units; unit += gridDim.x * 4) {
    const int b = unit / I, n = unit - b * I;
    const int expert = bk.expert[b], row0 = bk.row0[b], cnt = bk.cnt[b];
    const int slot = e2s ? e2s[expert] : expert;
    if (slot < 0 || slot >= w.num_slots) continue;  // the down kernel writes zero rows
    // row n of gate (m = 0) and up (m = 1): index words and codebooks
    const size_t row = (size_t)slot * I + n;
    uint3 q[2][kCbGU];
    uint4 cb[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* qr = (m == 0 ? w.qg : w.qu) + row * qrow;
      cb[m] = ld_cb((m == 0 ? w.cg : w.cu) + row * 8);
#pragma unroll
      for (int gi = 0; gi < kCbGU; ++gi) {
        const int G = lane + 64 * gi;
        q[m][gi] = G < NG ? ld12(qr + 12 * G) : make_uint3(0u, 0u, 0u);
      }
    }
    // the previous unit's table reads are done: a wavefront's LDS accesses complete in order
#pragma unroll
    for (int m = 0; m < 2; ++m) tab[m][lane] = cb3_table_entry(lane, cb[m]);
    __builtin_amdgcn_wave_barrier();
    for (int r = 0; r < cnt; ++r) {
      const uint16_t* xt = x + (size_t)(sorted_pair[row0 + r] / k) * H;
      float acc[2] = {0.f, 0.f};
#pragma unroll
      for (int gi = 0; gi < kCbGU; ++gi) {
        const int G = lane + 64 * gi;
        if (G >= NG) break;
        const uint4* px = reinterpret_cast<const uint4*>(xt + 32 * G);
        const uint4 xv[4] = {px[0], px[1], px[2], px[3]};
        const uint32_t xw[16] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w, xv[1].x, xv[1].y, xv[1].z, xv[1].w,
                                 xv[2].x, xv[2].y, xv[2].z, xv[2].w, xv[3].x, xv[3].y, xv[3].z, xv[3].w};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint32_t wv[16];
          cb3_group(q[m][gi], tab[m], wv);
          float a = acc[m];
#pragma unroll
          for (int t = 0; t < 16; ++t)
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv[t]),
                                                __builtin_bit_cast(bf16x2_t, xw[t]), a, false);
          acc[m] = a;
        }
      }
      // reduce (gate, up) over the wavefront: after the swap lanes 0-31 carry
      // gate partials and 32-63 up partials; the 16-lane sums of rows 0 + 1 and
      // 2 + 3 are added in that order
      const float a = sum16(tswap32(acc[0], acc[1]));
      const float gs = lane_value(a, 0) + lane_value(a, 16), us = lane_value(a, 32) + lane_value(a, 48);
      if (lane == 0) h[(size_t)(row0 + r) * I + n] = swiglu_f32(gs, us);
    }
  }
}

__global__ __launch_bounds__(kCbThreads, 2) void cb3_down_kernel(int k, int E, Cb3Store w,
                                                                 const int32_t* __restrict__ e2s,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ sorted_pair,
                                                                 const float* __restrict__ h, float* __restrict__ y) {
  __shared__ Buckets bk;
  __shared__ uint32_t tabs[4][4][64];  // per wavefront: the pair tables of its unit's four rows
  build_buckets(offsets, E, bk, nullptr);
  const int lane = threadIdx.x & 63;
  uint32_t (*tab)[64] = tabs[threadIdx.x >> 6];
  const int H = w.H, I = w.I, NG = I / 32;
  const size_t qrow = (size_t)I * 3 / 8;
  const int units = bk.n * (H / 4);
  for (int unit = blockIdx.x * 4 + (threadIdx.x >> 6); unit < units; unit += gridDim.x * 4) {
    const int b = unit / (H / 4), m0 = 4 * (unit - b * (H / 4));
    const int expert = bk.expert[b], row0 = bk.row0[b], cnt = bk.cnt[b];
    const int slot = e2s ? e2s[expert] : expert;
    if (slot < 0 || slot >= w.num_slots) {  // no stored expert: its rows are zero
      for (int r = 0; r < cnt; ++r)
        if (lane < 4) y[(size_t)sorted_pair[row0 + r] * H + m0 + lane] = 0.f;
      continue;
    }
    uint3 q[4][kCbDN];
    uint4 cb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t row = (size_t)slot * H + m0 + i;
      cb[i] = ld_cb(w.cd + row * 8);
#pragma unroll
      for (int gi = 0; gi < kCbDN; ++gi) {
        const int G = lane + 64 * gi;
        q[i][gi] = G < NG ? ld12(w.qd + row * qrow + 12 * G) : make_uint3(0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tab[i][lane] = cb3_table_entry(lane, cb[i]);
    __builtin_amdgcn_wave_barrier();
    for (int r = 0; r < cnt; ++r) {
      const float* hr = h + (size_t)(row0 + r) * I;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int gi = 0; gi < kCbDN; ++gi) {
        const int G = lane + 64 * gi;
        if (G >= NG) break;
        const float4_t* ph = reinterpret_cast<const float4_t*>(hr + 32 * G);
        float hv[32];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4_t t = ph[c];
          hv[4 * c] = t.x;
          hv[4 * c + 1] = t.y;
          hv[4 * c + 2] = t.z;
          hv[4 * c + 3] = t.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t wv[16];
          cb3_group(q[i][gi], tab[i], wv);
          float a = v[i];
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            a = fmaf(bf16_bits_to_f32(wv[t] & 0xFFFFu), hv[2 * t], a);
            a = fmaf(bf16_bits_to_f32(wv[t] >> 16), hv[2 * t + 1], a);
          }
          v[i] = a;
          __builtin_amdgcn_sched_barrier(0);  // one row's table reads live at a time
        }
      }
      // 4 row partials -> lane 16i holds the sum of row i
      const float a0 = tswap32(v[0], v[2]), a1 = tswap32(v[1], v[3]);
      const float c = sum16(tswap16(a0, a1));
      if ((lane & 15) == 0) y[(size_t)sorted_pair[row0 + r] * H + m0 + (lane >> 4)] = c;
    }
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
  hipLaunchKernelGGL(cb3_down_kernel, dim3(kCbGridDN), dim3(kCbThreads), 0, s, k, E, w, e2s, offsets, sorted_pair, h,
                     y_pair);
  return hipGetLastError();
}

}  // namespace moe
