// Streaming-read probe of the benchmark harness: reads a buffer once, every
// wavefront taking 16 consecutive KiB per step with one 16-byte load per lane
// per KiB (all 16 in flight), so that the read rate measured with it is the
// HBM ceiling that a well-coalesced streaming kernel can reach on this GPU.
// Also a clock probe (the shader clock while the GPU is busy) and a probe of
// the load shapes a weight tile can be read with.  Measurement only: nothing
// of the MoE arithmetic lives here.
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

// The same read with every KiB copied into the wavefront's LDS area by the
// buffer unit (buffer_load ... lds, 16 B a lane) instead of into registers:
// all 16 copies of a step in flight, then one word of the area read back.
__global__ __launch_bounds__(256) void stream_read_lds_kernel(const uint8_t* __restrict__ p, int64_t items,
                                                              unsigned* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t area[4][kDepth * 1024];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t wave = (int64_t)blockIdx.x * 4 + wid, nw = (int64_t)gridDim.x * 4;
  unsigned acc = 0;
  for (int64_t it = wave; it < items; it += nw) {
    // a resource over this step's 16 KiB: every offset below stays inside it
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p + it * (int64_t)kDepth * 1024), (short)0, (uint32_t)(kDepth * 1024), 0x00020000);
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(area[wid] + d * 1024), 16,
                                               (uint32_t)(d * 1024 + lane * 16), 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the step's copies are in LDS
    acc ^= *reinterpret_cast<const unsigned*>(area[wid] + ((int)(it % kDepth)) * 1024 + lane * 16);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): read before the next copies land
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
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

// Weight-tile load probe: the rate at which one CU pulls a weight tile's rows
// (512 rows x 2560 B, a gate/up tile's rows at hidden 5120) for the two load
// shapes a GEMM kernel can use, against where the rows live.  Workgroup b
// runs on XCD b % 8 and streams its own 512-row sets of that XCD's region
// (region_rows rows, so a region of 1.3 MB stays in the XCD's L2 and larger
// ones do not), NW wavefronts each with 32 loads of 1 KiB in flight per step:
//   PAT 0: 8 rows x 128 B per load (lane l: row l / 8, bytes 16 (l % 8) of
//          the row's 128-B chunk pair);
//   PAT 1: 32 rows x 32 B per load, the MFMA operand order of a 32-row
//          fragment (lane l: row l % 32, bytes 16 (l / 32) of the K-step);
//   PAT 2: 8 rows x 128 B per load with the lanes across rows (lane l: row
//          l % 8, bytes 16 (l / 8) of the chunk pair);
//   PAT 3: PAT 2's addresses copied into LDS by the buffer unit (16 B a lane),
//   PAT 4: PAT 0's addresses copied into LDS by the buffer unit;
//   PAT 5: PAT 0 with each row's eight 16-B pieces rotated by the row (lane l:
//          row l / 8, piece (l + l / 8) % 8), copied into LDS;
//   PAT 6: PAT 5's addresses into registers;
//   PAT 7: PAT 5 with half the copies in flight (NL = 64 / NW);
//   PAT 8: PAT 0 with 8 loads in flight;
// PAT 0-2 and 6 with 32 loads in flight per wavefront, PAT 3-5 with NL = 128 / NW
// (the LDS holds 128 KiB).  Every address lies inside the workgroup's region
// (rows wrap modulo region_rows, columns stay inside a 2560-B row), the loads
// go through a buffer resource bounded by the region, and every LDS copy
// lands inside the workgroup's array.
template <int PAT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void weight_load_probe_kernel(const uint8_t* __restrict__ buf,
                                                                       uint32_t region_rows, int iters,
                                                                       unsigned* __restrict__ sink) {
  constexpr bool kLds = (PAT >= 3 && PAT <= 5) || PAT == 7;
  constexpr int NL = PAT == 7 ? 64 / NW : PAT == 8 ? 8 : kLds ? 128 / NW : 32;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kLds ? NW * NL * 1024 : 16];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const size_t region_bytes = (size_t)region_rows * 2560u;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)(buf + xcd * region_bytes), (short)0,
                                                                     (uint32_t)region_bytes, 0x00020000);
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    const uint32_t c4 = (uint32_t)((it * 4) % 40);  // four 64-B chunks of K per step, 40 per row
    const uint32_t set = slot * (uint32_t)(NW / 4) + (uint32_t)(wid >> 2) + 32u * (NW / 4) * (uint32_t)(it / 10);
    const uint32_t row0 = (set * 512u) % region_rows;
    u4 v[kLds ? 1 : NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      uint32_t row, col;
      if (PAT == 0 || PAT == 4 || PAT == 8) {
        row = (uint32_t)(wid & 3) * 128u + (uint32_t)(j & 15) * 8u + (uint32_t)(lane >> 3);
        col = (c4 + 2u * (uint32_t)(j >> 4)) * 64u + (uint32_t)(lane & 7) * 16u;
      } else if (PAT == 5 || PAT == 6 || PAT == 7) {
        row = (uint32_t)(wid & 3) * 128u + (uint32_t)(j & 15) * 8u + (uint32_t)(lane >> 3);
        col = (c4 + 2u * (uint32_t)(j >> 4)) * 64u + (uint32_t)((lane + (lane >> 3)) & 7) * 16u;
      } else if (PAT == 1) {
        const uint32_t q = (uint32_t)(j & 7);
        row = (uint32_t)(wid & 3) * 128u + (q >> 1) * 32u + (uint32_t)(lane & 31);
        col = (c4 + (uint32_t)(j >> 3)) * 64u + (q & 1u) * 32u + (uint32_t)(lane >> 5) * 16u;
      } else {
        row = (uint32_t)(wid & 3) * 128u + (uint32_t)(j & 15) * 8u + (uint32_t)(lane & 7);
        col = (c4 + 2u * (uint32_t)(j >> 4)) * 64u + (uint32_t)(lane >> 3) * 16u;
      }
      const uint32_t off = ((row0 + row) % region_rows) * 2560u + col;
      if constexpr (kLds) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(stage + (wid * NL + j) * 1024), 16, off, 0, 0, 0);
      } else {
        v[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
      }
    }
    if constexpr (kLds) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's copies are in LDS
      const u4 w = *reinterpret_cast<const u4*>(stage + (wid * NL + (it % NL)) * 1024 + lane * 16);
      acc += w.x ^ (w.w * (unsigned)it);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): read before the next copies land
    } else {
#pragma unroll
      for (int j = 0; j < NL; ++j) acc += v[j].x ^ (v[j].w * (unsigned)j);
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads
}

}  // namespace

extern "C" {

// Launches the weight-tile load probe over 256 workgroups: buf holds 8 regions
// of region_rows rows of 2560 B; pattern 0-8; waves 4 or 8 per workgroup.
// Bytes read: 256 * iters * 1 KiB * (waves * 32 for patterns 0-2 and 6, 128
// for 3-5, 64 for 7, waves * 8 for 8).  0 on success, 1 on bad arguments, 2 on a launch error.
__attribute__((visibility("default"))) int gen_load_probe(const void* buf, int region_rows, int pattern, int waves,
                                                          int iters, void* sink, hipStream_t stream) {
  if (!buf || !sink || region_rows < 512 || (size_t)region_rows * 2560u >= 0x80000000u || iters <= 0 ||
      pattern < 0 || pattern > 8 || (waves != 4 && waves != 8))
    return 1;
  const dim3 g(256), b(64 * waves);
  const uint8_t* p = (const uint8_t*)buf;
  unsigned* k = (unsigned*)sink;
  const uint32_t rr = (uint32_t)region_rows;
  if (pattern == 0 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<0, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 0 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<0, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 1 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<1, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 1 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<1, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 2 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<2, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 2 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<2, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 3 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<3, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 3 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<3, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 4 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<4, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 4 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<4, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 5 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<5, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 5 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<5, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 6 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<6, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 6 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<6, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 7 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<7, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 7 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<7, 8>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 8 && waves == 4) hipLaunchKernelGGL((weight_load_probe_kernel<8, 4>), g, b, 0, stream, p, rr, iters, k);
  if (pattern == 8 && waves == 8) hipLaunchKernelGGL((weight_load_probe_kernel<8, 8>), g, b, 0, stream, p, rr, iters, k);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}


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

// gen_stream_read with the copies going into LDS (stream_read_lds_kernel).
__attribute__((visibility("default"))) int gen_stream_read_lds(const void* src, int64_t bytes, void* sink,
                                                               hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || bytes % (kDepth * 1024) != 0 || ((uintptr_t)src & 15u) != 0) return 1;
  hipLaunchKernelGGL(stream_read_lds_kernel, dim3(4096), dim3(256), 0, stream, (const uint8_t*)src,
                     bytes / (kDepth * 1024), (unsigned*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
