// Device filler for the synthetic expert weights: the SplitMix64 streams of
// gen/splitmix.py, evaluated on the GPU so that tens of GB of expert bytes can
// be produced in place.  SplitMix64 is the generator of Steele, Lea and Flood
// (OOPSLA 2014): out(n) = mix64(s0 + (n+1)*GAMMA), s0 = mix64(stream_id).
// Input generation only: nothing of the MoE arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t stream_seed(uint32_t seed, int layer, int expert, int matrix, int kind) {
  uint64_t id = ((uint64_t)seed << 32) | ((uint64_t)(layer & 0xFF) << 24) |
                ((uint64_t)(expert & 0xFFFF) << 8) | ((uint64_t)(matrix & 0xF) << 4) |
                (uint64_t)(kind & 0xF);
  return mix64(id);
}

// dst: [nslots][words_per_slot] u64; slot s holds expert slot_expert[s].
__global__ void fill_codes_kernel(uint64_t* __restrict__ dst, int64_t words_per_slot,
                                  const int32_t* __restrict__ slot_expert, uint32_t seed,
                                  int layer, int matrix) {
  const int slot = blockIdx.y;
  const uint64_t s0 = stream_seed(seed, layer, slot_expert[slot], matrix, 0);
  uint64_t* out = dst + (int64_t)slot * words_per_slot;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < words_per_slot; n += stride)
    out[n] = mix64(s0 + (uint64_t)(n + 1) * kGamma);
}

// dst: [nslots][bytes_per_slot] UE8M0 bytes, exponent uniform on [emin, 0].
__global__ void fill_scales_kernel(uint8_t* __restrict__ dst, int64_t bytes_per_slot,
                                   const int32_t* __restrict__ slot_expert, uint32_t seed,
                                   int layer, int matrix, int emin) {
  const int slot = blockIdx.y;
  const uint64_t s0 = stream_seed(seed, layer, slot_expert[slot], matrix, 1);
  const uint64_t nrange = (uint64_t)(1 - emin);
  uint8_t* out = dst + (int64_t)slot * bytes_per_slot;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < bytes_per_slot; n += stride) {
    uint64_t hi = mix64(s0 + (uint64_t)(n + 1) * kGamma) >> 32;
    out[n] = (uint8_t)(127 + emin + (int)((hi * nrange) >> 32));
  }
}

int grid_x(int64_t n, int nslots) {
  // enough blocks to cover ~4 waves of work per CU over all slots
  int64_t want = (n + 255) / 256;
  int64_t cap = (8192 + nslots - 1) / nslots;
  if (cap < 1) cap = 1;
  return (int)(want < cap ? (want < 1 ? 1 : want) : cap);
}

}  // namespace

extern "C" {

// Returns 0 on success, 1 on bad arguments, 2 on a launch error.
__attribute__((visibility("default"))) int gen_fill_codes(void* dst, int64_t bytes_per_slot, const int32_t* slot_expert_dev, int nslots,
                   uint32_t seed, int layer, int matrix, hipStream_t stream) {
  if (!dst || !slot_expert_dev || nslots <= 0 || nslots > 65535 || bytes_per_slot <= 0 ||
      bytes_per_slot % 8 != 0 || ((uintptr_t)dst & 7u) != 0)
    return 1;
  int64_t words = bytes_per_slot / 8;
  dim3 grid(grid_x(words, nslots), nslots);
  hipLaunchKernelGGL(fill_codes_kernel, grid, dim3(256), 0, stream, (uint64_t*)dst, words,
                     slot_expert_dev, seed, layer, matrix);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

__attribute__((visibility("default"))) int gen_fill_scales(void* dst, int64_t bytes_per_slot, const int32_t* slot_expert_dev, int nslots,
                    uint32_t seed, int layer, int matrix, int emin, hipStream_t stream) {
  if (!dst || !slot_expert_dev || nslots <= 0 || nslots > 65535 || bytes_per_slot <= 0 ||
      emin > 0 || emin < -127)
    return 1;
  dim3 grid(grid_x(bytes_per_slot, nslots), nslots);
  hipLaunchKernelGGL(fill_scales_kernel, grid, dim3(256), 0, stream, (uint8_t*)dst,
                     bytes_per_slot, slot_expert_dev, seed, layer, matrix, emin);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
