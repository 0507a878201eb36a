// Device helpers shared by the gfx950 kernels of the MXFP4 routed-expert FFN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int8_t_v __attribute__((ext_vector_type(8)));
typedef unsigned uint4_t __attribute__((ext_vector_type(4)));

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

}  // namespace moe
