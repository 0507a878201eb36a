// Fixed-order weighted slot sum and the weightless RMS norm (gfx950).
//
// Combine: the slot sum is its own kernel over rows that the expert FFN wrote
// once each ("DeepSeek V4.1 Flash Q4 / 27 September 2026", "30 September
// follow-up"), so the result does not depend on the order the experts ran in.
// Each thread owns four consecutive outputs of one token and accumulates the
// k slots in ascending j with fp32 FMAs; loads are 16-byte and coalesced, and
// eight slots' loads are in flight at once (slots past k re-read slot k-1 and
// are not added).
#include "common.cuh"
#include "kernels.h"

namespace moe {

namespace {

template <bool kBf16Out, bool kResidual>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      int k, int H, const uint16_t* __restrict__ res,
                                                      void* __restrict__ out) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  const float* wt = w + (size_t)t * k;
  const float* yt = y + (size_t)t * k * H + h;
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4_t v[8];
    float wj[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = min(j0 + i, k - 1);
      // streaming loads: each row is read once (at 4096 tokens 671 MB, far past the caches)
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(yt + (size_t)j * H));
      wj[i] = wt[j];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (j0 + i < k) {
        acc.x = fmaf(wj[i], v[i].x, acc.x);
        acc.y = fmaf(wj[i], v[i].y, acc.y);
        acc.z = fmaf(wj[i], v[i].z, acc.z);
        acc.w = fmaf(wj[i], v[i].w, acc.w);
      }
    }
  }
  if (kResidual) {
    const uint2 r = *reinterpret_cast<const uint2*>(res + (size_t)t * H + h);
    acc.x += bf16_bits_to_f32(r.x & 0xFFFFu);
    acc.y += bf16_bits_to_f32(r.x >> 16);
    acc.z += bf16_bits_to_f32(r.y & 0xFFFFu);
    acc.w += bf16_bits_to_f32(r.y >> 16);
  }
  if (kBf16Out) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H + h) = o;
  } else {
    *reinterpret_cast<float4_t*>(reinterpret_cast<float*>(out) + (size_t)t * H + h) = acc;
  }
}

// One workgroup per token: fp32 sum of squares (fixed reduction tree), then
// x / sqrt(mean + eps) rounded to bf16.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int H, float eps,
                                                      uint16_t* __restrict__ out) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const uint16_t* xt = x + (size_t)t * H;
  float ss = 0.f;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(xt + h);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_bits_to_f32(q[i] & 0xFFFFu), b = bf16_bits_to_f32(q[i] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = sqrtf(total / (float)H + eps);
  uint16_t* ot = out + (size_t)t * H;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(xt + h);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_bits_to_f32(q[i] & 0xFFFFu) / r, b = bf16_bits_to_f32(q[i] >> 16) / r;
      o[i] = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
    }
    *reinterpret_cast<uint4*>(ot + h) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_combine(const float* y_pair, const float* w, int T, int k, int H,
                          const uint16_t* residual, bool bf16_out, void* out, hipStream_t s) {
  dim3 grid((H + 1023) / 1024, T), block(256);
  if (bf16_out) {
    if (residual)
      hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, s, y_pair, w, k, H, residual, out);
    else
      hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, s, y_pair, w, k, H, residual, out);
  } else {
    if (residual)
      hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, s, y_pair, w, k, H, residual, out);
    else
      hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, s, y_pair, w, k, H, residual, out);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* x, int T, int H, float eps, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, s, x, H, eps, out);
  return hipGetLastError();
}

}  // namespace moe
