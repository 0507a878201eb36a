// Device helpers shared by the gfx950 kernels of the MXFP4 routed-expert FFN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int8_t_v __attribute__((ext_vector_type(8)));
typedef unsigned uint4_t __attribute__((ext_vector_type(4)));
typedef int i8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Sum over the 64 lanes of a wavefront; every lane receives the total.
// Butterfly order is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// UE8M0 byte -> 2^(e-127) as fp32, exact for every byte but 255
// (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// silu(g) * u in fp32: g * u / (1 + exp(-g)).
__device__ __forceinline__ float swiglu_f32(float g, float u) { return g * u / (1.0f + expf(-g)); }

// ---- cross-lane primitives without LDS (gfx9 DPP encodings, gfx950 permlane swaps)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16
constexpr int kDppRor8 = 0x128;       // lane i <- lane (i+8) mod 16 within 16

// Every lane gets the sum over its aligned group of 8 / 16 lanes.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  return v;
}
__device__ __forceinline__ float sum16(float v) { v = sum8(v); return v + dpp_mov<kDppMirror>(v); }

// Transposing reduction steps.  Each takes two per-lane partials a, b and
// returns one: the half (of the wave, of each 32-lane half, of each 16-lane
// row) named below carries a, the other b, each summed with its partner half.
//   tswap32: lanes 0-31 carry a, lanes 32-63 carry b
//   tswap16: rows 0 and 2 (lanes 0-15, 32-47) carry a, rows 1 and 3 carry b
//   tswap8 : lanes 0-7 of every row carry a, lanes 8-15 carry b
__device__ __forceinline__ float tswap32(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float tswap16(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float tswap8(float a, float b, int lane) {
  const float ar = dpp_mov<kDppRor8>(a), br = dpp_mov<kDppRor8>(b);
  return (lane & 8) ? b + br : a + ar;
}

// Every lane gets the sum over all 64 lanes (fixed combination order).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = sum16(v);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_mov_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Every lane gets the maximum over all 64 lanes.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_mov_u64<kDppXor1>(v));
  v = umax64(v, dpp_mov_u64<kDppXor2>(v));
  v = umax64(v, dpp_mov_u64<kDppHalfMirror>(v));
  v = umax64(v, dpp_mov_u64<kDppMirror>(v));
  {
    auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = umax64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
  }
  {
    auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = umax64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
  }
  return v;
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// ---- buffer-resource loads ---------------------------------------------------------
//
// A wave-uniform base and byte range; an offset past the range reads zeros.
// Rows beyond a bucket's end get such an offset, so every load of the K loop
// is issued unconditionally and the compiler can count the loads in flight
// exactly (a load behind a branch makes it wait for all of them).

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw 32-bit access, range-checked
constexpr uint32_t kOob = 0x80000000u;         // an offset past every range used here

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), (int)kRsrcWord3);
}

__device__ __forceinline__ uint4_t bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// The same with the non-temporal cache policy, for bytes read once per call.
__device__ __forceinline__ uint4_t bload16_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
}

// Rows 0-15 (P) and 16-31 (Q) as loaded, 16-lane groups [b0 b1 b2 b3] of 16
// rows each  ->  K-step 0 = [P.b0 Q.b0 P.b1 Q.b1], K-step 1 = [P.b2 Q.b2 P.b3 Q.b3]
// (lane l: row l%32, block 2s + l/32).
__device__ __forceinline__ void b_operands(const uint4_t& P, const uint4_t& Q, i8v& s0, i8v& s1) {
  uint32_t o0[4], o1[4];
  const uint32_t p[4] = {P.x, P.y, P.z, P.w}, q[4] = {Q.x, Q.y, Q.z, Q.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const auto t = __builtin_amdgcn_permlane16_swap(p[d], q[d], false, false);   // [P0 Q0 P2 Q2], [P1 Q1 P3 Q3]
    const auto u = __builtin_amdgcn_permlane32_swap(t[0], t[1], false, false);   // [P0 Q0 P1 Q1], [P2 Q2 P3 Q3]
    o0[d] = u[0];
    o1[d] = u[1];
  }
  s0 = i8v{(int)o0[0], (int)o0[1], (int)o0[2], (int)o0[3], 0, 0, 0, 0};
  s1 = i8v{(int)o1[0], (int)o1[1], (int)o1[2], (int)o1[3], 0, 0, 0, 0};
}

// Words [cw0, cw0 + WIN) of ROWS scale-table rows, in two steps so that their
// latency overlaps the first chunk loads of the K loop: issue() loads into
// registers, store() writes the table.  row_off(r) is the byte offset of row
// r's scale bytes (kOob for rows past the bucket).
template <int ROWS, int NT, int WIN, int STRIDE>  // STRIDE: words per table row
struct ScaleRows {
  static constexpr int N = ROWS * WIN / NT;
  static_assert(ROWS * WIN % NT == 0 && WIN < STRIDE, "table split");
  uint32_t v[N];
  template <typename RowOff>
  __device__ __forceinline__ void issue(rsrc_t r, int cw0, int t, RowOff row_off) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = t + NT * i, row = idx / WIN, wd = idx - row * WIN;
      const uint32_t o = row_off(row);
      v[i] = bload4(r, o == kOob ? kOob : o + 4u * (uint32_t)(cw0 + wd));
    }
  }
  __device__ __forceinline__ void store(uint32_t* tab, int t) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = t + NT * i, row = idx / WIN, wd = idx - row * WIN;
      tab[row * STRIDE + wd] = v[i];
    }
  }
  // The same words in chunk-major order for 128 rows: word wd of row r at
  // (32 wd + r % 32) * 4 + r / 32, so one 16-byte read returns the words of
  // rows r32, r32 + 32, r32 + 64 and r32 + 96 for one chunk.
  __device__ __forceinline__ void store_cf(uint32_t* tab, int t) const {
    static_assert(ROWS == 128, "four 32-row fragments");
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = t + NT * i, row = idx / WIN, wd = idx - row * WIN;
      tab[(32 * wd + (row & 31)) * 4 + (row >> 5)] = v[i];
    }
  }
};

// Compact list of the non-empty buckets, built by wavefront 0 into LDS.  With
// a run mask ([E] bytes, nonzero: run now) only the buckets of masked-in
// experts are listed, so every other bucket's rows are left untouched.
struct Buckets {
  int n;
  int expert[kMaxExperts];
  int row0[kMaxExperts];
  int cnt[kMaxExperts];
};

__device__ inline void build_buckets(const int32_t* __restrict__ offsets, int E, Buckets& b,
                                     const uint8_t* __restrict__ run) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    constexpr int CH = kMaxExperts / 64;
    int off[CH + 1];
    bool on[CH];
#pragma unroll
    for (int i = 0; i <= CH; ++i) {
      const int e = lane * CH + i;
      off[i] = offsets[e < E ? e : E];
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = lane * CH + i;
      on[i] = e < E && off[i + 1] > off[i] && (run == nullptr || run[e] != 0);
    }
    int n = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) n += on[i] ? 1 : 0;
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
      if (on[i]) {
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

}  // namespace moe
