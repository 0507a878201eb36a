// C ABI of the MXFP4 routed-expert FFN: argument validation, then enqueue.
// Every check here runs before any HIP call, so a rejected call touches
// neither the device nor the stream.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_fp4.h"
#include "kernels.h"

namespace {

inline bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// The int a C caller passed for an enum argument, read without loading an
// out-of-range value as the enum type; checked against the named values.
template <typename Enum>
int enum_bits(const Enum* e) {
  static_assert(sizeof(Enum) == sizeof(int), "C enums are int-sized");
  int v;
  memcpy(&v, e, sizeof v);
  return v;
}

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

moe_status check_store(const moe_fp4_experts* w) {
  if (!w) return MOE_ERR_NULL;
  if (!w->w_gate || !w->s_gate || !w->w_up || !w->s_up || !w->w_down || !w->s_down) return MOE_ERR_NULL;
  if (w->num_slots < 1 || w->hidden < 256 || w->inter < 128) return MOE_ERR_SHAPE;
  if (w->hidden % 256 != 0 || w->inter % 128 != 0) return MOE_ERR_SHAPE;
  if (w->hidden > 16384 || w->inter > 8192) return MOE_ERR_UNSUPPORTED;
  if (misaligned(w->w_gate, 16) || misaligned(w->w_up, 16) || misaligned(w->w_down, 16)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe::ExpertStore to_store(const moe_fp4_experts* w) {
  return moe::ExpertStore{w->num_slots, w->hidden, w->inter, w->w_gate, w->s_gate,
                          w->w_up,      w->s_up,   w->w_down, w->s_down};
}

moe_status check_ffn_common(const uint16_t* x, int32_t T, int32_t k, int32_t E, const moe_fp4_experts* w,
                            const int32_t* e2s, const int32_t* offsets, const int32_t* sorted_pair,
                            float* y_pair, void* ws, size_t ws_bytes, size_t need) {
  moe_status st = check_store(w);
  if (st != MOE_OK) return st;
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS || k > E) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !offsets || !sorted_pair || !y_pair) return MOE_ERR_NULL;
  if (!e2s && w->num_slots < E) return MOE_ERR_SHAPE;
  if (misaligned(x, 16) || misaligned(y_pair, 16)) return MOE_ERR_ALIGN;
  if (need > 0) {
    if (!ws) return MOE_ERR_WORKSPACE;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (misaligned(ws, 256)) return MOE_ERR_ALIGN;
  }
  return MOE_OK;
}

// Scratch of moe_decode_layer_noalloc: a device array of the library, so
// that call needs no allocation.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device (with that device current) and only that address is handed to the
// kernels.  Every call on one device shares that device's copy.
__device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`; false if the runtime cannot give it.
bool noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return false;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return true;
}

}  // namespace

extern "C" {

MOE_FP4_API const char* moe_status_string(moe_status s) {
  switch (enum_bits(&s)) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_ALIGN: return "a pointer misses its required alignment";
    case MOE_ERR_UNSUPPORTED: return "shape not supported by this library";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

MOE_FP4_API moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                                 const int32_t* expert_to_slot, int32_t* topk_ids, float* topk_w,
                                 hipStream_t stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E) return MOE_ERR_SHAPE;
  if ((int64_t)T * E > INT32_MAX) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_NULL;
  return launched(moe::launch_route(logits, T, E, k, expert_to_slot, topk_ids, topk_w, stream));
}

static moe_status check_router_gate(const uint16_t* x_bf16, int32_t T, int32_t hidden, const uint16_t* w_router,
                                    int32_t E, const float* logits) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (hidden < 256 || hidden % 256 != 0 || hidden > 16384) return MOE_ERR_SHAPE;
  if ((int64_t)T * E > INT32_MAX) return MOE_ERR_SHAPE;
  if ((int64_t)T * hidden * 2 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;  // 31-bit buffer offsets
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w_router || !logits) return MOE_ERR_NULL;
  if (misaligned(x_bf16, 16) || misaligned(w_router, 16)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

MOE_FP4_API moe_status moe_router_logits(const uint16_t* x_bf16, int32_t T, int32_t hidden,
                                         const uint16_t* w_router, int32_t E, const float* bias, float* logits,
                                         hipStream_t stream) {
  const moe_status st = check_router_gate(x_bf16, T, hidden, w_router, E, logits);
  if (st != MOE_OK || T == 0) return st;
  return launched(moe::launch_router_logits(x_bf16, T, hidden, w_router, E, bias, logits, stream));
}

MOE_FP4_API moe_status moe_route_x(const uint16_t* x_bf16, int32_t T, int32_t hidden, const uint16_t* w_router,
                                   int32_t E, const float* bias, int32_t k, const int32_t* expert_to_slot,
                                   float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  if (k < 1 || k > MOE_MAX_TOPK || k > E) return MOE_ERR_SHAPE;
  const moe_status st = check_router_gate(x_bf16, T, hidden, w_router, E, logits);
  if (st != MOE_OK || T == 0) return st;
  if (!topk_ids || !topk_w) return MOE_ERR_NULL;
  return launched(moe::launch_route_x(x_bf16, T, hidden, w_router, E, bias, k, expert_to_slot, logits, topk_ids,
                                      topk_w, stream));
}

MOE_FP4_API size_t moe_ffn_cb3_decode_workspace_bytes(int32_t T, int32_t k, int32_t inter) {
  if (T < 0 || k < 1 || inter < 1) return 0;
  return moe::decode_workspace_bytes(T, k, inter);
}

MOE_FP4_API moe_status moe_ffn_cb3_decode(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                          const moe_cb3_experts* w, const int32_t* expert_to_slot,
                                          const int32_t* expert_offsets, const int32_t* sorted_pair,
                                          float* y_pair, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!w) return MOE_ERR_NULL;
  if (!w->q_gate || !w->q_up || !w->q_down || !w->cb_gate || !w->cb_up || !w->cb_down) return MOE_ERR_NULL;
  if (w->num_slots < 1 || w->hidden < 256 || w->inter < 128) return MOE_ERR_SHAPE;
  if (w->hidden % 256 != 0 || w->inter % 128 != 0) return MOE_ERR_SHAPE;
  if (!moe::cb3_decode_supported(w->hidden, w->inter)) return MOE_ERR_UNSUPPORTED;
  if (misaligned(w->q_gate, 4) || misaligned(w->q_up, 4) || misaligned(w->q_down, 4)) return MOE_ERR_ALIGN;
  if (misaligned(w->cb_gate, 16) || misaligned(w->cb_up, 16) || misaligned(w->cb_down, 16)) return MOE_ERR_ALIGN;
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS || k > E) return MOE_ERR_SHAPE;
  if (T > MOE_DECODE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !expert_offsets || !sorted_pair || !y_pair) return MOE_ERR_NULL;
  if (!expert_to_slot && w->num_slots < E) return MOE_ERR_SHAPE;
  if (misaligned(x_bf16, 16) || misaligned(y_pair, 16)) return MOE_ERR_ALIGN;
  const size_t need = moe::decode_workspace_bytes(T, k, w->inter);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (misaligned(ws, 256)) return MOE_ERR_ALIGN;
  const moe::Cb3Store st{w->num_slots, w->hidden, w->inter, w->q_gate, w->q_up, w->q_down,
                         w->cb_gate, w->cb_up, w->cb_down};
  return launched(moe::launch_decode_cb3(x_bf16, T, k, E, st, expert_to_slot, expert_offsets, sorted_pair, y_pair, ws,
                                         stream));
}

MOE_FP4_API size_t moe_permute_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || (int64_t)T * k > (1 << 24)) return 0;  // moe_permute rejects more pairs
  return moe::permute_workspace_bytes(T * k, E);
}

MOE_FP4_API moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                                   int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_to_row,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if ((int64_t)T * k > (1 << 24)) return MOE_ERR_SHAPE;
  if (!expert_offsets) return MOE_ERR_NULL;
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_to_row)) return MOE_ERR_NULL;
  const size_t need = moe::permute_workspace_bytes(T * k, E);
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (need > 0 && misaligned(ws, 256)) return MOE_ERR_ALIGN;
  // T == 0 still enqueues: the offsets of an empty batch are all zero.
  return launched(moe::launch_permute(topk_ids, T * k, E, expert_offsets, sorted_pair, pair_to_row, ws, stream));
}

MOE_FP4_API size_t moe_ffn_fp4_decode_workspace_bytes(int32_t T, int32_t k, int32_t inter) {
  if (T < 0 || k < 1 || inter < 1) return 0;
  return moe::decode_workspace_bytes(T, k, inter);
}

static moe_status decode_phase(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E, const moe_fp4_experts* w,
                               const int32_t* expert_to_slot, const int32_t* expert_offsets,
                               const int32_t* sorted_pair, float* y_pair, void* ws, size_t ws_bytes, int phase,
                               hipStream_t stream, const uint8_t* run = nullptr, bool invariant = false) {
  if (T > MOE_DECODE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  const size_t need = (T > 0 && k > 0 && w) ? moe::decode_workspace_bytes(T, k, w->inter) : 0;
  moe_status st = check_ffn_common(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, y_pair,
                                   ws, ws_bytes, need);
  if (st != MOE_OK || T == 0) return st;
  if (invariant)  // every batch size on the multi-token kernels, whose rows do not depend on the batch
    return launched(moe::launch_decode_mt(x_bf16, T, k, E, to_store(w), expert_to_slot, expert_offsets,
                                          sorted_pair, y_pair, ws, phase, stream, run));
  return launched(moe::launch_decode(x_bf16, T, k, E, to_store(w), expert_to_slot, expert_offsets,
                                     sorted_pair, y_pair, ws, phase, stream, run));
}

MOE_FP4_API moe_status moe_ffn_fp4_decode(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                          const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                          const int32_t* expert_offsets, const int32_t* sorted_pair,
                                          float* y_pair, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_phase(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, y_pair, ws, ws_bytes, 0,
                      stream);
}

MOE_FP4_API moe_status moe_ffn_fp4_decode_invariant(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                    const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                    const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                    float* y_pair, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_phase(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, y_pair, ws, ws_bytes, 0,
                      stream, nullptr, true);
}

MOE_FP4_API moe_status moe_ffn_fp4_decode_subset(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                 const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                 const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                 const uint8_t* run_mask, float* y_pair, void* ws, size_t ws_bytes,
                                                 hipStream_t stream) {
  if (!run_mask && T > 0) return MOE_ERR_NULL;
  return decode_phase(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, y_pair, ws, ws_bytes, 0,
                      stream, run_mask);
}

MOE_FP4_API moe_status moe_ffn_fp4_decode_gateup(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                 const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                 const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                 float* y_pair, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_phase(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, y_pair, ws, ws_bytes, 1,
                      stream);
}

MOE_FP4_API moe_status moe_ffn_fp4_decode_down(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                               const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                               const int32_t* expert_offsets, const int32_t* sorted_pair,
                                               float* y_pair, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_phase(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, y_pair, ws, ws_bytes, 2,
                      stream);
}

namespace {

struct LayerWs {
  int32_t *offsets, *sorted_pair, *pair_to_row;
  void* pws;
  void* hws;
  float* y;
  size_t total;
};

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

// Offsets are computed first and turned into pointers only for a real base
// (a size query passes none: no arithmetic on a null pointer).
LayerWs layer_ws_layout(int T, int k, int E, int H, int I, void* base) {
  const size_t P = (size_t)T * k;
  const int Pi = P > (size_t)INT32_MAX ? INT32_MAX : (int)P;
  size_t off = up256((size_t)(E + 1) * 4);
  const size_t o_sp = off;
  off += up256(P * 4);
  const size_t o_p2r = off;
  off += up256(P * 4);
  const size_t o_pws = off;
  off += up256(moe::permute_workspace_bytes(Pi, E));
  const size_t o_hws = off;
  off += up256(moe::decode_workspace_bytes(T, k, I));
  const size_t o_y = off;
  off += up256(P * H * 4);
  LayerWs l{};
  l.total = off;
  if (base) {
    uint8_t* p = reinterpret_cast<uint8_t*>(base);
    l.offsets = reinterpret_cast<int32_t*>(p);
    l.sorted_pair = reinterpret_cast<int32_t*>(p + o_sp);
    l.pair_to_row = reinterpret_cast<int32_t*>(p + o_p2r);
    l.pws = p + o_pws;
    l.hws = p + o_hws;
    l.y = reinterpret_cast<float*>(p + o_y);
  }
  return l;
}

}  // namespace

MOE_FP4_API size_t moe_decode_layer_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t hidden, int32_t inter) {
  if (T < 1 || k < 1 || E < 1 || hidden < 1 || inter < 1) return 0;
  if (moe::fused_decode_supported(T, k, E, hidden, inter)) return moe::fused_decode_workspace_bytes(k, inter);
  return layer_ws_layout(T, k, E, hidden, inter, nullptr).total;
}

// Checks of a decode-layer call other than its workspace; *need receives the
// workspace bytes the call takes.  MOE_OK with *need == 0 means T == 0 (nothing to do).
static moe_status check_decode_layer(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E, int32_t k,
                                     const int32_t* expert_to_slot, const moe_fp4_experts* w,
                                     const uint16_t* residual_bf16, int od, const void* out,
                                     const int32_t* topk_ids, const float* topk_w, bool norm, float eps,
                                     size_t* need) {
  *need = 0;
  if (T > MOE_DECODE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  if (od != MOE_OUT_BF16 && od != MOE_OUT_F32) return MOE_ERR_UNSUPPORTED;
  moe_status st = check_store(w);
  if (st != MOE_OK) return st;
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS || k > E) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!logits || !x_bf16 || !out || !topk_ids || !topk_w) return MOE_ERR_NULL;
  if (!expert_to_slot && w->num_slots < E) return MOE_ERR_SHAPE;
  if (misaligned(x_bf16, 16) || misaligned(out, 16) || (residual_bf16 && misaligned(residual_bf16, 16)))
    return MOE_ERR_ALIGN;
  if (norm && !(eps >= 0.0f)) return MOE_ERR_SHAPE;
  const size_t lbytes = moe_decode_layer_workspace_bytes(T, k, E, w->hidden, w->inter);
  *need = norm ? up256(lbytes) + up256((size_t)T * w->hidden * 2) : lbytes;
  return MOE_OK;
}

// norm: x_bf16 is the raw residual row; it is normalised first (as moe_rmsnorm_bf16, eps) and is
// itself the residual (residual_bf16 is then ignored).
static moe_status decode_layer(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E, int32_t k,
                               const int32_t* expert_to_slot, const moe_fp4_experts* w, const uint16_t* residual_bf16,
                               int od, void* out, int32_t* topk_ids, float* topk_w, void* ws,
                               size_t ws_bytes, int phase, hipStream_t stream, bool norm = false, float eps = 0.f) {
  size_t need = 0;
  const moe_status st = check_decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, residual_bf16, enum_bits(&od), out,
                                           topk_ids, topk_w, norm, eps, &need);
  if (st != MOE_OK || T == 0) return st;
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (misaligned(ws, 256)) return MOE_ERR_ALIGN;
  const size_t lbytes = moe_decode_layer_workspace_bytes(T, k, E, w->hidden, w->inter);
  const moe::ExpertStore store = to_store(w);
  const bool bf16 = od == MOE_OUT_BF16;
  if (norm) residual_bf16 = x_bf16;
  if (moe::fused_decode_supported(T, k, E, w->hidden, w->inter))
    return launched(moe::launch_decode_fused(logits, x_bf16, E, k, expert_to_slot, store, residual_bf16, bf16, out,
                                             topk_ids, topk_w, ws, phase, stream, norm, eps));
  const LayerWs l = layer_ws_layout(T, k, E, w->hidden, w->inter, ws);
  hipError_t e = hipSuccess;
  if (norm) {  // the normalised rows after the layer's own workspace
    uint16_t* n = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(ws) + up256(lbytes));
    if (phase != 2) e = moe::launch_rmsnorm(x_bf16, T, w->hidden, eps, n, stream);
    x_bf16 = n;
  }
  if (phase != 2) {
    e = moe::launch_route(logits, T, E, k, expert_to_slot, topk_ids, topk_w, stream);
    if (e == hipSuccess)
      e = moe::launch_permute(topk_ids, T * k, E, l.offsets, l.sorted_pair, l.pair_to_row, l.pws, stream);
    if (e == hipSuccess)
      e = moe::launch_decode(x_bf16, T, k, E, store, expert_to_slot, l.offsets, l.sorted_pair, l.y, l.hws, 1, stream);
  }
  if (phase != 1) {
    if (e == hipSuccess)
      e = moe::launch_decode(x_bf16, T, k, E, store, expert_to_slot, l.offsets, l.sorted_pair, l.y, l.hws, 2, stream);
    if (e == hipSuccess) e = moe::launch_combine(l.y, topk_w, T, k, w->hidden, residual_bf16, bf16, out, stream);
  }
  return launched(e);
}

MOE_FP4_API moe_status moe_decode_layer(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E, int32_t k,
                                        const int32_t* expert_to_slot, const moe_fp4_experts* w,
                                        const uint16_t* residual_bf16, moe_out_dtype od, void* out,
                                        int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  return decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, residual_bf16, enum_bits(&od), out, topk_ids, topk_w, ws,
                      ws_bytes, 0, stream);
}

MOE_FP4_API size_t moe_decode_layer_invariant_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t hidden,
                                                              int32_t inter) {
  if (T < 1 || k < 1 || E < 1 || hidden < 1 || inter < 1) return 0;
  if (T == 1) return moe::invariant_layer_workspace_bytes(k, hidden, inter);
  return layer_ws_layout(T, k, E, hidden, inter, nullptr).total;
}

MOE_FP4_API moe_status moe_decode_layer_invariant(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                                  int32_t k, const int32_t* expert_to_slot, const moe_fp4_experts* w,
                                                  const uint16_t* residual_bf16, moe_out_dtype od, void* out,
                                                  int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                                                  hipStream_t stream) {
  size_t need = 0;
  const moe_status st = check_decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, residual_bf16, enum_bits(&od), out,
                                           topk_ids, topk_w, false, 0.f, &need);
  if (st != MOE_OK || T == 0) return st;
  need = moe_decode_layer_invariant_workspace_bytes(T, k, E, w->hidden, w->inter);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (misaligned(ws, 256)) return MOE_ERR_ALIGN;
  const moe::ExpertStore store = to_store(w);
  const bool bf16 = od == MOE_OUT_BF16;
  if (T == 1)
    return launched(moe::launch_invariant_layer(logits, x_bf16, E, k, expert_to_slot, store, residual_bf16, bf16,
                                                out, topk_ids, topk_w, ws, stream));
  const LayerWs l = layer_ws_layout(T, k, E, w->hidden, w->inter, ws);
  hipError_t e = moe::launch_route(logits, T, E, k, expert_to_slot, topk_ids, topk_w, stream);
  if (e == hipSuccess)
    e = moe::launch_permute(topk_ids, T * k, E, l.offsets, l.sorted_pair, l.pair_to_row, l.pws, stream);
  if (e == hipSuccess)
    e = moe::launch_decode_mt(x_bf16, T, k, E, store, expert_to_slot, l.offsets, l.sorted_pair, l.y, l.hws, 0,
                              stream);
  if (e == hipSuccess) e = moe::launch_combine(l.y, topk_w, T, k, w->hidden, residual_bf16, bf16, out, stream);
  return launched(e);
}

MOE_FP4_API moe_status moe_decode_layer_noalloc(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                                int32_t k, const int32_t* expert_to_slot, const moe_fp4_experts* w,
                                                const uint16_t* residual_bf16, moe_out_dtype od, void* out,
                                                int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  size_t need = 0;
  const moe_status st = check_decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, residual_bf16, enum_bits(&od), out,
                                           topk_ids, topk_w, false, 0.f, &need);
  if (st != MOE_OK || T == 0) return st;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (!noalloc_scratch(&ws)) return MOE_ERR_LAUNCH;
  return decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, residual_bf16, enum_bits(&od), out, topk_ids, topk_w, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, 0, stream);
}

MOE_FP4_API moe_status moe_decode_layer_gateup(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                               int32_t k, const int32_t* expert_to_slot, const moe_fp4_experts* w,
                                               const uint16_t* residual_bf16, moe_out_dtype od, void* out,
                                               int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                                               hipStream_t stream) {
  return decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, residual_bf16, enum_bits(&od), out, topk_ids, topk_w, ws,
                      ws_bytes, 1, stream);
}

MOE_FP4_API moe_status moe_decode_layer_down(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                             int32_t k, const int32_t* expert_to_slot, const moe_fp4_experts* w,
                                             const uint16_t* residual_bf16, moe_out_dtype od, void* out,
                                             int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
  return decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, residual_bf16, enum_bits(&od), out, topk_ids, topk_w, ws,
                      ws_bytes, 2, stream);
}

MOE_FP4_API size_t moe_decode_layer_rmsnorm_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t hidden,
                                                            int32_t inter) {
  if (T <= 0 || k <= 0 || hidden <= 0) return 0;
  return up256(moe_decode_layer_workspace_bytes(T, k, E, hidden, inter)) + up256((size_t)T * hidden * 2);
}

MOE_FP4_API moe_status moe_decode_layer_rmsnorm(const float* logits, const uint16_t* x_bf16, float eps, int32_t T,
                                                int32_t E, int32_t k, const int32_t* expert_to_slot,
                                                const moe_fp4_experts* w, moe_out_dtype od, void* out,
                                                int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                                                hipStream_t stream) {
  return decode_layer(logits, x_bf16, T, E, k, expert_to_slot, w, nullptr, enum_bits(&od), out, topk_ids, topk_w, ws, ws_bytes,
                      0, stream, true, eps);
}

MOE_FP4_API size_t moe_ffn_fp4_prefill_workspace_bytes(int32_t T, int32_t k, int32_t hidden, int32_t inter) {
  if (T < 0 || k < 1 || hidden < 1 || inter < 1) return 0;
  return moe::prefill_workspace_bytes(T, k, hidden, inter);
}

static moe_status prefill_call(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E, const moe_fp4_experts* w,
                               const int32_t* expert_to_slot, const int32_t* expert_offsets,
                               const int32_t* sorted_pair, int act, float* y_pair, void* ws,
                               size_t ws_bytes, hipStream_t stream, const uint8_t* run,
                               const uint8_t* packed = nullptr) {
  if (act != MOE_ACT_MXFP6_E2M3) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * k > (1 << 22)) return MOE_ERR_SHAPE;
  // the MXFP6 activations (x once per sorted row, and h) are addressed with 31-bit buffer offsets
  if (w && T > 0 && k > 0 &&
      ((int64_t)T * k * (w->hidden / 32) * 24 >= ((int64_t)1 << 31) ||
       (int64_t)T * k * (w->inter / 32) * 24 >= ((int64_t)1 << 31)))
    return MOE_ERR_UNSUPPORTED;
  if (w && (misaligned(w->s_gate, 4) || misaligned(w->s_up, 4) || misaligned(w->s_down, 4))) return MOE_ERR_ALIGN;
  const size_t need = (T > 0 && k > 0 && w) ? moe::prefill_workspace_bytes(T, k, w->hidden, w->inter) : 0;
  moe_status st = check_ffn_common(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, y_pair,
                                   ws, ws_bytes, need);
  if (st != MOE_OK || T == 0) return st;
  return launched(moe::launch_prefill(x_bf16, T, k, E, to_store(w), expert_to_slot, expert_offsets,
                                      sorted_pair, y_pair, ws, stream, run, packed));
}

MOE_FP4_API moe_status moe_ffn_fp4_prefill(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                           const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                           const int32_t* expert_offsets, const int32_t* sorted_pair,
                                           moe_act_fmt act, float* y_pair, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  return prefill_call(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, enum_bits(&act), y_pair, ws, ws_bytes,
                      stream, nullptr);
}

MOE_FP4_API size_t moe_prefill_packed_bytes(int32_t num_slots, int32_t hidden, int32_t inter) {
  if (num_slots < 1 || hidden < 256 || hidden % 256 != 0 || inter < 128 || inter % 128 != 0) return 0;
  return moe::prefill_packed_bytes(num_slots, hidden, inter);
}

MOE_FP4_API moe_status moe_prefill_pack_weights(const moe_fp4_experts* w, void* packed, size_t packed_bytes,
                                                hipStream_t stream) {
  moe_status st = check_store(w);
  if (st != MOE_OK) return st;
  if (!packed) return MOE_ERR_NULL;
  if (w->hidden % 256 != 0 || w->inter % 128 != 0) return MOE_ERR_SHAPE;
  if (misaligned(packed, 256)) return MOE_ERR_ALIGN;
  if (packed_bytes < moe::prefill_packed_bytes(w->num_slots, w->hidden, w->inter)) return MOE_ERR_WORKSPACE;
  // a slot's blocks are addressed with 32-bit offsets
  if (moe_prefill_packed_bytes(1, w->hidden, w->inter) >= ((size_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return launched(moe::launch_pack_weights(to_store(w), static_cast<uint8_t*>(packed), stream));
}

MOE_FP4_API moe_status moe_ffn_fp4_prefill_packed(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                  const moe_fp4_experts* w, const void* packed, size_t packed_bytes,
                                                  const int32_t* expert_to_slot, const int32_t* expert_offsets,
                                                  const int32_t* sorted_pair, moe_act_fmt act, float* y_pair,
                                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T > 0) {
    if (!packed) return MOE_ERR_NULL;
    if (!w) return MOE_ERR_NULL;
    if (misaligned(packed, 256)) return MOE_ERR_ALIGN;
    if (w->num_slots > 0 && packed_bytes < moe::prefill_packed_bytes(w->num_slots, w->hidden, w->inter))
      return MOE_ERR_WORKSPACE;
    if (moe::prefill_packed_bytes(1, w->hidden, w->inter) >= ((size_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  }
  return prefill_call(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, enum_bits(&act), y_pair, ws, ws_bytes,
                      stream, nullptr, static_cast<const uint8_t*>(packed));
}

MOE_FP4_API moe_status moe_ffn_fp4_prefill_subset(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                  const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                  const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                  const uint8_t* run_mask, moe_act_fmt act, float* y_pair, void* ws,
                                                  size_t ws_bytes, hipStream_t stream) {
  if (!run_mask && T > 0) return MOE_ERR_NULL;
  return prefill_call(x_bf16, T, k, E, w, expert_to_slot, expert_offsets, sorted_pair, enum_bits(&act), y_pair, ws, ws_bytes,
                      stream, run_mask);
}

MOE_FP4_API moe_status moe_combine(const float* y_pair, const float* topk_w, int32_t T, int32_t k, int32_t H,
                                   const uint16_t* residual_bf16, moe_out_dtype od, void* out,
                                   hipStream_t stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  const int odv = enum_bits(&od);
  if (odv != MOE_OUT_BF16 && odv != MOE_OUT_F32) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_pair || !topk_w || !out) return MOE_ERR_NULL;
  if (misaligned(y_pair, 16) || misaligned(out, 16) || (residual_bf16 && misaligned(residual_bf16, 16)))
    return MOE_ERR_ALIGN;
  if (T > 65535) return MOE_ERR_UNSUPPORTED;
  return launched(moe::launch_combine(y_pair, topk_w, T, k, H, residual_bf16, odv == MOE_OUT_BF16, out, stream));
}

MOE_FP4_API moe_status moe_rmsnorm_bf16(const uint16_t* x_bf16, int32_t T, int32_t H, float eps,
                                        uint16_t* out_bf16, hipStream_t stream) {
  if (T < 0 || H < 8 || H % 8 != 0 || H > 65536 || !(eps >= 0.0f)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !out_bf16) return MOE_ERR_NULL;
  if (misaligned(x_bf16, 16) || misaligned(out_bf16, 16)) return MOE_ERR_ALIGN;
  return launched(moe::launch_rmsnorm(x_bf16, T, H, eps, out_bf16, stream));
}

}  // extern "C"
