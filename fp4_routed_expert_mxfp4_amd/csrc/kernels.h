// Internal launchers of the gfx950 kernels; the C ABI in api.cpp validates
// arguments and then calls these.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

struct ExpertStore {
  int num_slots, H, I;
  const uint8_t *wg, *sg, *wu, *su, *wd, *sd;
};

hipError_t launch_route(const float* logits, int T, int E, int k, const int32_t* e2s, int32_t* ids,
                        float* w, hipStream_t s);

// Router gate projection logits = x . W_r^T (+ bias): bf16 x and W_r [E][H],
// fp32 logits [T][E].  launch_route_x then routes the written logits
// (launch_route).
hipError_t launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias,
                                float* logits, hipStream_t s);
hipError_t launch_route_x(const uint16_t* x, int T, int H, const uint16_t* wr, int E, const float* bias, int k,
                          const int32_t* e2s, float* logits, int32_t* ids, float* tw, hipStream_t s);

size_t permute_workspace_bytes(int P, int E);
hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_to_row, void* ws, hipStream_t s);

// Decode FFN: gate/up + SwiGLU into h (sorted-row order, in ws), then down.
size_t decode_workspace_bytes(int T, int k, int I);
// phase: 0 both kernels, 1 gate/up only, 2 down only.  run: [E] bytes, or NULL
// for every expert; the buckets of experts whose byte is 0 are skipped and
// their y rows left as they are.
hipError_t launch_decode(const uint16_t* x, int T, int k, int E, const ExpertStore& w,
                         const int32_t* e2s, const int32_t* offsets, const int32_t* sorted_pair,
                         float* y_pair, void* ws, int phase, hipStream_t s, const uint8_t* run = nullptr);

// Multi-token decode FFN (bf16 MFMA); launch_decode uses it for every shape
// the one-token kernels do not cover.  ws holds h as bf16 hi and lo planes.
hipError_t launch_decode_mt(const uint16_t* x, int T, int k, int E, const ExpertStore& w, const int32_t* e2s,
                            const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws, int phase,
                            hipStream_t s, const uint8_t* run = nullptr);

// The batch-invariant decode layer of one token in one call (route + gate/up,
// down, combine) on the multi-token kernels' arithmetic.
size_t invariant_layer_workspace_bytes(int k, int H, int I);
hipError_t launch_invariant_layer(const float* logits, const uint16_t* x, int E, int k, const int32_t* e2s,
                                  const ExpertStore& w, const uint16_t* residual, bool bf16_out, void* out,
                                  int32_t* topk_ids, float* topk_w, void* ws, hipStream_t s);

// Fused one-token decode layer (route + gate/up, then down + combine).
bool fused_decode_supported(int T, int k, int E, int H, int I);
size_t fused_decode_workspace_bytes(int k, int I);
// norm: x is the raw residual row; K1 normalises it (as launch_rmsnorm does, bit
// for bit) before the gate/up projection.
hipError_t launch_decode_fused(const float* logits, const uint16_t* x, int E, int k, const int32_t* e2s,
                               const ExpertStore& w, const uint16_t* residual, bool bf16_out, void* out,
                               int32_t* topk_ids, float* topk_w, void* ws, int phase, hipStream_t s,
                               bool norm = false, float eps = 0.f);

// Prefill FFN on block-scaled MFMA with MXFP6 activations.  packed: the
// experts' copy in MFMA operand order (launch_pack_weights) for the tiled
// GEMMs, or null to read the row-major store.
size_t prefill_workspace_bytes(int T, int k, int H, int I);
hipError_t launch_prefill(const uint16_t* x, int T, int k, int E, const ExpertStore& w,
                          const int32_t* e2s, const int32_t* offsets, const int32_t* sorted_pair,
                          float* y_pair, void* ws, hipStream_t s, const uint8_t* run = nullptr,
                          const uint8_t* packed = nullptr);
size_t prefill_packed_bytes(int num_slots, int H, int I);
hipError_t launch_pack_weights(const ExpertStore& w, uint8_t* dst, hipStream_t s);

// Decode FFN over experts in the 3-bit per-row codebook format: index bytes
// [S][rows][K*3/8], codebooks [S][rows][8] bf16; h fp32 in ws as for launch_decode.
struct Cb3Store {
  int num_slots, H, I;
  const uint8_t *qg, *qu, *qd;
  const uint16_t *cg, *cu, *cd;
};
bool cb3_decode_supported(int H, int I);
hipError_t launch_decode_cb3(const uint16_t* x, int T, int k, int E, const Cb3Store& w, const int32_t* e2s,
                             const int32_t* offsets, const int32_t* sorted_pair, float* y_pair, void* ws,
                             hipStream_t s);

hipError_t launch_combine(const float* y_pair, const float* w, int T, int k, int H,
                          const uint16_t* residual, bool bf16_out, void* out, hipStream_t s);

hipError_t launch_rmsnorm(const uint16_t* x, int T, int H, float eps, uint16_t* out, hipStream_t s);

}  // namespace moe
