// Streaming-read probe of the benchmark harness: reads a buffer once, every
// wavefront taking 16 consecutive KiB per step with one 16-byte load per lane
// per KiB (all 16 in flight), so that the read rate measured with it is the
// HBM ceiling that a well-coalesced streaming kernel can reach on this GPU.
// Also a clock probe (the shader clock while the GPU is busy).  Measurement
// only: nothing of the MoE arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u4 __attribute__((ext_vector_type(4)));
constexpr int kDepth = 16;  // KiB per wavefront step

__global__ __launch_bounds__(256) void stream_read_kernel(const u4* __restrict__ p, int64_t items,
                                                          unsigned* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), nw = (int64_t)gridDim.x * 4;
  unsigned acc = 0;
  for (int64_t it = wave; it < items; it += nw) {
    const u4* b = p + it * kDepth * 64 + lane;
    u4 v[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) v[d] = __builtin_nontemporal_load(b + d * 64);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; no byte pattern used here gives this value
}

// Shader clock against the constant 100 MHz clock: every workgroup (one
// wavefront) reads both counters, runs `iters` dependent multiply-adds and
// reads them again; out[2b] and out[2b + 1] receive workgroup b's two deltas.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, int iters) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  float v = (float)threadIdx.x;
  for (int i = 0; i < iters; ++i) v = __builtin_fmaf(v, 0.999999f, 0.5f);
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (v == -1.0f) out[0] = 0;  // keeps the loop; v stays positive
}

}  // namespace

extern "C" {

// Launches the clock probe: blocks workgroups of one wavefront; out holds
// 2 * blocks words.  0 on success, 1 on bad arguments, 2 on a launch error.
__attribute__((visibility("default"))) int gen_clock_probe(void* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks <= 0 || blocks > 4096 || iters <= 0) return 1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(64), 0, stream, (uint64_t*)out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads bytes (a multiple of 16 KiB) at src (16-byte aligned) once.  sink: a
// device word the kernel may write.  0 on success, 1 on bad arguments, 2 on a
// launch error.
__attribute__((visibility("default"))) int gen_stream_read(const void* src, int64_t bytes, void* sink,
                                                           hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || bytes % (kDepth * 1024) != 0 || ((uintptr_t)src & 15u) != 0) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(4096), dim3(256), 0, stream, (const u4*)src, bytes / (kDepth * 1024),
                     (unsigned*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
