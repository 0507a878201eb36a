// Drives every entry point of include/moe_fp4.h through its argument
// validation and workspace arithmetic, for the sanitizer build of the C-ABI
// layer (AddressSanitizer and UndefinedBehaviorSanitizer on the host code).
// It runs without a GPU: pointers are aligned fake addresses that validation
// never dereferences, and a call that passes validation reaches a kernel
// launch, which fails without a device (MOE_ERR_LAUNCH) or succeeds on one.
// Exit status 0 when every call returned what the header documents.
#include <stdint.h>
#include <stdio.h>

#include <climits>

#include "moe_fp4.h"

namespace {

int g_fail = 0;

void expect(const char* what, int line, moe_status got, moe_status want) {
  if (got != want) {
    printf("line %d: %s returned %d, expected %d\n", line, what, (int)got, (int)want);
    ++g_fail;
  }
}

// A call that passes validation: it then launches, which fails without a GPU.
void expect_valid(const char* what, int line, moe_status got) {
  if (got != MOE_OK && got != MOE_ERR_LAUNCH) {
    printf("line %d: %s returned %d, expected a launch\n", line, what, (int)got);
    ++g_fail;
  }
}

#define EXPECT(call, want) expect(#call, __LINE__, (call), (want))
#define VALID(call) expect_valid(#call, __LINE__, (call))

template <typename T>
T* fake(uintptr_t a = 0x100000) {
  return reinterpret_cast<T*>(a);
}

moe_fp4_experts store(int slots, int hidden, int inter) {
  moe_fp4_experts w{};
  w.num_slots = slots;
  w.hidden = hidden;
  w.inter = inter;
  w.w_gate = fake<uint8_t>(0x200000);
  w.s_gate = fake<uint8_t>(0x300000);
  w.w_up = fake<uint8_t>(0x400000);
  w.s_up = fake<uint8_t>(0x500000);
  w.w_down = fake<uint8_t>(0x600000);
  w.s_down = fake<uint8_t>(0x700000);
  return w;
}

}  // namespace

int main() {
  const float* lg = fake<const float>();
  const uint16_t* x = fake<const uint16_t>();
  int32_t* ids = fake<int32_t>();
  float* tw = fake<float>();
  void* ws = fake<void>(0x800000);
  const size_t big = (size_t)1 << 40;
  const hipStream_t st = nullptr;
  moe_fp4_experts w = store(384, 5120, 2304);
  moe_fp4_experts ws8 = store(8, 1024, 256);

  // workspace queries at the extremes of every argument: no overflow, no UB
  for (int32_t T : {0, 1, 16, 4096, 1 << 20, INT32_MAX})
    for (int32_t k : {1, 8, 16})
      for (int32_t E : {1, 384, 1024}) {
        (void)moe_permute_workspace_bytes(T, k, E);
        (void)moe_ffn_fp4_decode_workspace_bytes(T, k, 8192);
        (void)moe_decode_layer_workspace_bytes(T, k, E, 16384, 8192);
        (void)moe_decode_layer_invariant_workspace_bytes(T, k, E, 16384, 8192);
        (void)moe_decode_layer_rmsnorm_workspace_bytes(T, k, E, 16384, 8192);
        (void)moe_ffn_fp4_prefill_workspace_bytes(T, k, 16384, 8192);
        (void)moe_ffn_cb3_decode_workspace_bytes(T, k, 8192);
      }
  for (int s = 0; s < 8; ++s) (void)moe_status_string((moe_status)s);

  // router
  VALID(moe_route(lg, 4096, 384, 8, nullptr, ids, tw, st));
  EXPECT(moe_route(nullptr, 1, 384, 8, nullptr, ids, tw, st), MOE_ERR_NULL);
  EXPECT(moe_route(lg, 1, 384, 17, nullptr, ids, tw, st), MOE_ERR_SHAPE);
  EXPECT(moe_route(lg, 1, 4, 8, nullptr, ids, tw, st), MOE_ERR_SHAPE);
  EXPECT(moe_route(lg, INT32_MAX, 1024, 16, nullptr, ids, tw, st), MOE_ERR_SHAPE);
  EXPECT(moe_route(lg, 0, 384, 8, nullptr, nullptr, nullptr, st), MOE_OK);

  // router gate projection
  VALID(moe_router_logits(x, 16, 5120, fake<const uint16_t>(), 384, nullptr, fake<float>(), st));
  VALID(moe_route_x(x, 16, 5120, fake<const uint16_t>(), 384, nullptr, 8, nullptr, fake<float>(), ids, tw, st));
  EXPECT(moe_route_x(x, 16, 5120, nullptr, 384, nullptr, 8, nullptr, fake<float>(), ids, tw, st), MOE_ERR_NULL);
  EXPECT(moe_route_x(x, 16, 5121, fake<const uint16_t>(), 384, nullptr, 8, nullptr, fake<float>(), ids, tw, st),
         MOE_ERR_SHAPE);

  // bucketing
  int32_t* off = fake<int32_t>(0x900000);
  VALID(moe_permute(ids, 4096, 8, 384, off, ids, ids, ws, big, st));
  EXPECT(moe_permute(ids, 4096, 8, 384, off, ids, ids, nullptr, 0, st), MOE_ERR_WORKSPACE);
  EXPECT(moe_permute(ids, INT32_MAX, 16, 384, off, ids, ids, ws, big, st), MOE_ERR_SHAPE);
  EXPECT(moe_permute(ids, 1, 8, 384, nullptr, ids, ids, ws, big, st), MOE_ERR_NULL);

  // decode FFN calls
  float* y = fake<float>(0xA00000);
  VALID(moe_ffn_fp4_decode(x, 1, 8, 384, &w, nullptr, off, ids, y, ws, big, st));
  VALID(moe_ffn_fp4_decode_invariant(x, 16, 8, 384, &w, nullptr, off, ids, y, ws, big, st));
  VALID(moe_ffn_fp4_decode_gateup(x, 1, 8, 384, &w, nullptr, off, ids, y, ws, big, st));
  VALID(moe_ffn_fp4_decode_down(x, 1, 8, 384, &w, nullptr, off, ids, y, ws, big, st));
  VALID(moe_ffn_fp4_decode_subset(x, 16, 8, 384, &w, nullptr, off, ids, fake<const uint8_t>(), y, ws, big, st));
  EXPECT(moe_ffn_fp4_decode(x, 1, 8, 384, &w, nullptr, off, ids, y, ws, 16, st), MOE_ERR_WORKSPACE);
  EXPECT(moe_ffn_fp4_decode(x, 300, 8, 384, &w, nullptr, off, ids, y, ws, big, st), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_ffn_fp4_decode(fake<const uint16_t>(0x100002), 1, 8, 384, &w, nullptr, off, ids, y, ws, big, st),
         MOE_ERR_ALIGN);
  moe_fp4_experts bad = store(384, 5000, 2304);
  EXPECT(moe_ffn_fp4_decode(x, 1, 8, 384, &bad, nullptr, off, ids, y, ws, big, st), MOE_ERR_SHAPE);
  EXPECT(moe_ffn_fp4_decode(x, 1, 8, 384, nullptr, nullptr, off, ids, y, ws, big, st), MOE_ERR_NULL);

  // decode layers
  void* out = fake<void>(0xB00000);
  VALID(moe_decode_layer(lg, x, 1, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, ws, big, st));
  VALID(moe_decode_layer(lg, x, 16, 384, 8, nullptr, &w, x, MOE_OUT_F32, out, ids, tw, ws, big, st));
  VALID(moe_decode_layer_invariant(lg, x, 1, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, ws, big, st));
  VALID(moe_decode_layer_invariant(lg, x, 16, 384, 8, nullptr, &w, nullptr, MOE_OUT_F32, out, ids, tw, ws, big, st));
  VALID(moe_decode_layer_gateup(lg, x, 1, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, ws, big, st));
  VALID(moe_decode_layer_down(lg, x, 1, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, ws, big, st));
  VALID(moe_decode_layer_rmsnorm(lg, x, 1e-6f, 1, 384, 8, nullptr, &w, MOE_OUT_BF16, out, ids, tw, ws, big, st));
  VALID(moe_decode_layer_noalloc(lg, x, 1, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, st));
  EXPECT(moe_decode_layer_noalloc(lg, x, 256, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, st),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_decode_layer(lg, x, 1, 384, 8, nullptr, &w, nullptr, (moe_out_dtype)7, out, ids, tw, ws, big, st),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_decode_layer_invariant(lg, x, 1, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, ws, 64, st),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_decode_layer_rmsnorm(lg, x, -1.0f, 1, 384, 8, nullptr, &w, MOE_OUT_BF16, out, ids, tw, ws, big, st),
         MOE_ERR_SHAPE);
  EXPECT(moe_decode_layer(lg, x, INT32_MAX, 384, 8, nullptr, &w, nullptr, MOE_OUT_BF16, out, ids, tw, ws, big, st),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_decode_layer(lg, x, 1, 8, 2, nullptr, &ws8, nullptr, MOE_OUT_BF16, out, ids, tw,
                          fake<void>(0x800010), big, st),
         MOE_ERR_ALIGN);

  // prefill
  VALID(moe_ffn_fp4_prefill(x, 4096, 8, 384, &w, nullptr, off, ids, MOE_ACT_MXFP6_E2M3, y, ws, big, st));
  VALID(moe_ffn_fp4_prefill_subset(x, 4096, 8, 384, &w, nullptr, off, ids, fake<const uint8_t>(), MOE_ACT_MXFP6_E2M3,
                                   y, ws, big, st));
  EXPECT(moe_ffn_fp4_prefill(x, 4096, 8, 384, &w, nullptr, off, ids, (moe_act_fmt)3, y, ws, big, st),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_ffn_fp4_prefill(x, INT32_MAX, 16, 384, &w, nullptr, off, ids, MOE_ACT_MXFP6_E2M3, y, ws, big, st),
         MOE_ERR_SHAPE);
  EXPECT(moe_ffn_fp4_prefill(x, 4096, 8, 384, &w, nullptr, off, ids, MOE_ACT_MXFP6_E2M3, y, ws, 4096, st),
         MOE_ERR_WORKSPACE);

  // cb3 decode
  moe_cb3_experts c{};
  c.num_slots = 384;
  c.hidden = 5120;
  c.inter = 2304;
  c.q_gate = c.q_up = c.q_down = fake<uint8_t>(0xC00000);
  c.cb_gate = c.cb_up = c.cb_down = fake<uint16_t>(0xD00000);
  VALID(moe_ffn_cb3_decode(x, 1, 8, 384, &c, nullptr, off, ids, y, ws, big, st));
  EXPECT(moe_ffn_cb3_decode(x, 1, 8, 384, nullptr, nullptr, off, ids, y, ws, big, st), MOE_ERR_NULL);

  // combine and norm
  VALID(moe_combine(y, tw, 4096, 8, 5120, nullptr, MOE_OUT_BF16, out, st));
  EXPECT(moe_combine(y, tw, 4096, 8, 5121, nullptr, MOE_OUT_BF16, out, st), MOE_ERR_SHAPE);
  VALID(moe_rmsnorm_bf16(x, 16, 5120, 1e-6f, fake<uint16_t>(0xE00000), st));
  EXPECT(moe_rmsnorm_bf16(x, 16, 5120, -1.0f, fake<uint16_t>(0xE00000), st), MOE_ERR_SHAPE);

  printf("%s: %d mismatches\n", g_fail ? "FAIL" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
