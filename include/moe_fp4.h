/*
 * moe_fp4.h -- C ABI of the routed Mixture-of-Experts FFN over MXFP4 experts
 * on AMD Instinct MI355X (gfx950).
 *
 * The method is the routed-expert FFN of a DeepSeek-V4.1-Flash-class model as
 * the pages describe it:
 *   - every routed expert is three matrices (gate, up: [I][H]; down: [H][I])
 *     stored as e2m1 codes with one UE8M0 scale per 32 weights -- "DeepSeek-
 *     V4.1-Flash on a single NVIDIA DGX Spark", "Why it is built this way"
 *     (15,360 experts x 3 x 2304 x 5120 weights at FP4 + UE8M0/32) and its
 *     intro (the checkpoint's own e2m1 experts, never requantised);
 *   - only a kept subset of the experts may be routable -- same page, "The
 *     numbers" (the top ~40 % of experts stay routable and resident);
 *   - each (token, slot) pair gets its own output row, produced exactly
 *     once, and adding a token's rows together is its own pass in a fixed
 *     order -- "DeepSeek V4.1 Flash Q4 / 27 September 2026", "30 September
 *     follow-up: prefill" (why its two-wave MoE is bit-exact);
 *   - prefill and decode are separate arithmetic paths, each judged against
 *     its own reference -- "Fast single-box DeepSeek v4.1 Flash runtime",
 *     "Conventions".
 *
 * Conventions shared by every call
 * ---------------------------------
 *  - Array arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees, synchronises or reads device memory back on the
 *    host.  The one exception is `const moe_fp4_experts* w`, a HOST pointer to
 *    a small struct that itself holds device pointers; it is read during the
 *    call only.
 *  - Each call validates its arguments synchronously.  On failure it returns
 *    a status and enqueues nothing.  On success it enqueues its kernels on
 *    `stream` and returns at once; a launch failure is reported as
 *    MOE_ERR_LAUNCH.  No call prints, throws or keeps global mutable state.
 *  - No call records a memset, so every call may be captured into a HIP graph.
 *  - Element layouts are row-major.  e2m1 codes are packed two per byte,
 *    element 2c in the low nibble of byte c.  A scale byte e stands for
 *    2^(e-127), every byte 0..254 being valid.  Byte 255 (NaN in the OCP MX
 *    encoding) must not occur; it is not checked on the device, and rows
 *    that use it come out non-finite (the one-token decode kernels read it
 *    as +inf, the MFMA kernels as NaN).  The one-token decode kernels scale
 *    each block sum in fp32 (byte 0 is the fp32 subnormal 2^-127); the
 *    multi-token decode kernels fold the scale into bf16 weights, exact for
 *    every weight of magnitude 2^-126 or more, so bytes 0-2 may round their
 *    smallest weights; the prefill kernels pass the byte to the MFMA.
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - Device data are not inspected on the host.  Preconditions on their
 *    contents (finite logits, expert ids in range, at least k routable
 *    experts) are documented per call; when they are violated the kernels
 *    still stay inside every buffer, but the values written are unspecified.
 *  - T == 0 is valid everywhere; it enqueues nothing, except moe_permute,
 *    which still writes the E+1 zero offsets of the empty batch.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FP4_API __attribute__((visibility("default")))

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL                         */
  MOE_ERR_SHAPE = 2,        /* a size is out of range or inconsistent             */
  MOE_ERR_ALIGN = 3,        /* a pointer misses the alignment stated for it       */
  MOE_ERR_UNSUPPORTED = 4,  /* a valid shape this library has no kernel for       */
  MOE_ERR_WORKSPACE = 5,    /* workspace missing or smaller than the query says   */
  MOE_ERR_LAUNCH = 6        /* the HIP runtime rejected a kernel launch           */
} moe_status;

typedef enum { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1 } moe_out_dtype;

/* Activation encoding of the prefill path (MX block format, 32 per scale). */
typedef enum { MOE_ACT_MXFP6_E2M3 = 0 } moe_act_fmt;

/* One layer's expert store, the checkpoint's own layout, indexed by slot.
 * Slot s holds one expert; expert_to_slot tables map expert ids to slots.
 *   w_gate, w_up : [num_slots][inter][hidden/2]  e2m1 codes  (16-byte aligned)
 *   s_gate, s_up : [num_slots][inter][hidden/32] UE8M0 bytes
 *   w_down       : [num_slots][hidden][inter/2]  e2m1 codes  (16-byte aligned)
 *   s_down       : [num_slots][hidden][inter/32] UE8M0 bytes
 * Rows are the output features; K (the reduction index) is contiguous.
 * Requirements: hidden % 256 == 0, inter % 128 == 0, hidden <= 16384,
 * inter <= 8192, num_slots >= 1.  One expert occupies
 * 3*hidden*inter/2 + 3*hidden*inter/32 bytes (18,800,640 B at 5120 x 2304,
 * the "18.8 MB" per-expert read of the DGX Spark page, "Open WebUI"). */
typedef struct {
  int32_t num_slots, hidden, inter;
  const uint8_t *w_gate, *s_gate;
  const uint8_t *w_up, *s_up;
  const uint8_t *w_down, *s_down;
} moe_fp4_experts;

/* Limits of this library. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
#define MOE_DECODE_MAX_TOKENS 256

/* ---------------------------------------------------------------------------
 * moe_route -- top-k router.
 * The pages give no scoring function; the reading implemented is: for token
 * t, the candidates are the experts e with expert_to_slot[e] >= 0 (all
 * experts when expert_to_slot is NULL) -- the kept/routable subset of the DGX
 * Spark page, "The numbers".  Candidates are ordered by (logit descending,
 * expert index ascending); slot j receives rank j; weights are the softmax of
 * the k selected logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), in fp32.
 *   logits         [T][E] fp32, finite (NaN is treated as -inf)
 *   expert_to_slot [E] int32 or NULL
 *   topk_ids       [T][k] int32 out: expert ids
 *   topk_w         [T][k] fp32  out
 * 1 <= k <= MOE_MAX_TOPK, k <= E <= MOE_MAX_EXPERTS.  If fewer than k experts
 * are routable, the remaining slots get non-routable experts with weight 0.
 * ------------------------------------------------------------------------- */
MOE_FP4_API moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                                 const int32_t* expert_to_slot, int32_t* topk_ids,
                                 float* topk_w, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_router_logits -- the router's gate projection, the step before moe_route.
 * The router runs before any expert can be read: prefill could stage only the
 * experts "the router selected", which waits on the layer's router ("DeepSeek
 * V4.1 Flash Q4 / 27 September 2026", "30 September follow-up: prefill"; the
 * split router of its "4 October follow-up").  The pages give neither its
 * form nor its precision; the reading implemented is the plain linear gate
 *   logits[t][e] = sum_c x[t][c] * w_router[e][c] + bias[e]
 * with bf16 x and W_r (every product exact in fp32) and fp32 sums in a fixed
 * order, so the logits are run-to-run deterministic.  Up to 64 tokens run as
 * a GEMV (one workgroup per expert row), larger batches as a bf16 MFMA GEMM.
 *   x_bf16   [T][hidden] bf16 bits (16-byte aligned)
 *   w_router [E][hidden] bf16 bits (16-byte aligned), row e = expert e
 *   bias     [E] fp32 or NULL (added after the dot product)
 *   logits   [T][E] fp32 out
 * hidden % 256 == 0, 256 <= hidden <= 16384, 1 <= E <= MOE_MAX_EXPERTS,
 * T*hidden*2 < 2^31 (else MOE_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------- */
MOE_FP4_API moe_status moe_router_logits(const uint16_t* x_bf16, int32_t T, int32_t hidden,
                                         const uint16_t* w_router, int32_t E, const float* bias,
                                         float* logits, hipStream_t stream);

/* moe_route_x -- moe_router_logits followed by moe_route in one call: the
 * gate projection and the top-k with the routable subset of moe_route.
 * logits (required, [T][E] fp32) receives the projected logits; topk_ids and
 * topk_w are exactly what moe_route writes for those logits (the router
 * kernel runs on them after the projection).  Arguments and limits: as
 * moe_router_logits and moe_route. */
MOE_FP4_API moe_status moe_route_x(const uint16_t* x_bf16, int32_t T, int32_t hidden, const uint16_t* w_router,
                                   int32_t E, const float* bias, int32_t k, const int32_t* expert_to_slot,
                                   float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_permute -- token-to-expert bucketing of the (token, slot) rows.
 * Pair p = t*k + j.  expert_offsets[e] = number of pairs routed to experts
 * below e (exclusive prefix sum of the per-expert counts; expert_offsets[E] =
 * T*k).  sorted_pair lists every p ordered by (expert ascending, p ascending)
 * -- a stable, order-independent bucketing, so the expert FFN can run the
 * experts in any order ("30 September follow-up: prefill" of the 27 September
 * argonautlabs report).  pair_to_row is the inverse permutation.
 *   topk_ids       [T*k] int32, each in [0, E)
 *   expert_offsets [E+1] int32 out
 *   sorted_pair    [T*k] int32 out
 *   pair_to_row    [T*k] int32 out
 *   ws             device workspace of moe_permute_workspace_bytes(T, k, E)
 *                  bytes, 256-byte aligned (may be NULL when that is 0, which
 *                  it is for T*k <= 1024)
 * T*k <= 2^24.  Ids outside [0, E) are left out of every bucket (their
 * pair_to_row entry is -1 and expert_offsets[E] counts only valid pairs;
 * sorted rows from expert_offsets[E] on are not written).  The expert FFN
 * calls read and write nothing for such a pair: its y_pair row keeps what it
 * held, and moe_combine adds that row like any other.
 * ------------------------------------------------------------------------- */
MOE_FP4_API size_t moe_permute_workspace_bytes(int32_t T, int32_t k, int32_t E);
MOE_FP4_API moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                                   int32_t* expert_offsets, int32_t* sorted_pair,
                                   int32_t* pair_to_row, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_ffn_fp4_decode -- expert FFN of the decode path (fp32 accumulation).
 * Decode is a weight stream: a token reads its k experts once, and the
 * M5 Max engine's decode kernels run at 69-100 % of its memory roofline
 * ("DeepSeek V4.1 Flash Q4 / 27 September 2026", "28 September follow-up"),
 * so every weight byte is loaded once with 16-byte coalesced reads and
 * decoded in registers.  Decode is judged against unquantised activations
 * ("Fast single-box DeepSeek v4.1 Flash runtime", "Conventions").
 * For every pair p = sorted_pair[r] = t*k + j with expert e (bucket of r):
 *   g = W_gate[e] . x_t,  u = W_up[e] . x_t,  h = silu(g) * u  (fp32),
 *   y_pair[p] = W_down[e] . h                                  (fp32)
 * where W = e2m1(code) * 2^(scale-127) is decoded in registers.  x is used as
 * given (bf16, exact in fp32) and h keeps fp32 precision: this is the decode
 * reference arithmetic, judged against unquantised activations.  One token at
 * hidden = 1024*J (J <= 6) with inter/32 = 64*M + 8*tail (M <= 1) runs on VALU
 * dot products; every other call (two or more tokens, other shapes) on bf16
 * MFMA with h carried as bf16 hi + lo (relative error <= 2^-18), where a
 * token's rows are bit-identical whichever tokens share the batch.
 *   x_bf16         [T][hidden] bf16 bits (16-byte aligned)
 *   expert_to_slot [E] int32 (NULL: slot = expert id, needs num_slots >= E);
 *                  a bucket whose expert has no slot (-1 or >= num_slots)
 *                  writes zero rows
 *   expert_offsets [E+1], sorted_pair [T*k]: outputs of moe_permute
 *   y_pair         [T*k][hidden] fp32 out, row p (token-slot order)
 *   ws             device workspace of at least
 *                  moe_ffn_fp4_decode_workspace_bytes(T, k, inter) bytes,
 *                  256-byte aligned; contents on entry do not matter
 * A token may name one expert in several of its slots (topk_ids from
 * moe_route never do); every such pair gets its own, equal, y_pair row.
 * 1 <= T <= MOE_DECODE_MAX_TOKENS.
 * ------------------------------------------------------------------------- */
MOE_FP4_API size_t moe_ffn_fp4_decode_workspace_bytes(int32_t T, int32_t k, int32_t inter);
MOE_FP4_API moe_status moe_ffn_fp4_decode(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                          const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                          const int32_t* expert_offsets, const int32_t* sorted_pair,
                                          float* y_pair, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/* moe_ffn_fp4_decode_invariant -- moe_ffn_fp4_decode with every batch size on
 * the multi-token (bf16 MFMA, h as hi + lo) arithmetic, so that a token's
 * y_pair rows are bit-identical whether it is decoded alone or inside a batch
 * (a verify round of speculative decoding): the single-box runtime's
 * verification reproduces single-token decode bit for bit, and its hardest
 * bugs were batched-versus-single disagreements ("Fast single-box DeepSeek
 * v4.1 Flash runtime", "Dependency order and swarm split"; exact multi-row
 * kernels, "Document map").  Same arguments and workspace as
 * moe_ffn_fp4_decode; one token costs more than on the one-token kernels. */
MOE_FP4_API moe_status moe_ffn_fp4_decode_invariant(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                    const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                    const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                    float* y_pair, void* ws, size_t ws_bytes,
                                                    hipStream_t stream);

/* moe_ffn_fp4_decode_gateup, moe_ffn_fp4_decode_down -- the two kernels of
 * moe_ffn_fp4_decode as separate calls with the same arguments: gateup writes
 * h (sorted-row order) into the workspace, down reads it from there
 * and writes y_pair.  gateup followed by down on one stream, with the same
 * workspace, is exactly moe_ffn_fp4_decode.  They let a caller time or
 * schedule the two weight streams separately. */
MOE_FP4_API moe_status moe_ffn_fp4_decode_gateup(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                 const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                 const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                 float* y_pair, void* ws, size_t ws_bytes,
                                                 hipStream_t stream);
MOE_FP4_API moe_status moe_ffn_fp4_decode_down(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                               const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                               const int32_t* expert_offsets, const int32_t* sorted_pair,
                                               float* y_pair, void* ws, size_t ws_bytes,
                                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_decode_layer -- one whole decode layer: moe_route, moe_permute,
 * moe_ffn_fp4_decode and moe_combine in one call, with the same results bit
 * for bit.  Kernel boundaries cost a measurable share of a decode token
 * ("DeepSeek V4.1 Flash Q4 / 27 September 2026", "28 September follow-up":
 * 3-5 ms of command-buffer boundaries in a 43 ms token); for one token
 * (T == 1, k <= 8, hidden a multiple of 1024 up to 6144, inter = 2048*M or
 * 2048*M + 256 with M <= 1) the layer runs as two kernels: route + gate/up,
 * then down + the fixed-order slot sum written straight to `out`.  Other
 * shapes run the four steps with their intermediates in the workspace.
 *   logits [T][E] fp32, x_bf16 [T][hidden] bf16 (16-byte aligned),
 *   expert_to_slot, w: as for moe_route and moe_ffn_fp4_decode
 *   residual_bf16 [T][hidden] or NULL; od, out [T][hidden]: as moe_combine
 *   topk_ids [T][k], topk_w [T][k]: the routing (outputs, as moe_route)
 *   ws: moe_decode_layer_workspace_bytes(T, k, E, hidden, inter) bytes,
 *       256-byte aligned; contents on entry do not matter
 * 1 <= T <= MOE_DECODE_MAX_TOKENS.
 * ------------------------------------------------------------------------- */
MOE_FP4_API size_t moe_decode_layer_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t hidden,
                                                    int32_t inter);
MOE_FP4_API moe_status moe_decode_layer(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                        int32_t k, const int32_t* expert_to_slot,
                                        const moe_fp4_experts* w, const uint16_t* residual_bf16,
                                        moe_out_dtype od, void* out, int32_t* topk_ids, float* topk_w,
                                        void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_decode_layer_invariant -- one whole decode layer (route, bucketing,
 * expert FFN, combine) in one call on the batch-invariant arithmetic of
 * moe_ffn_fp4_decode_invariant: the output and topk_ids/topk_w are
 * bit-identical to moe_route, moe_permute, moe_ffn_fp4_decode_invariant and
 * moe_combine, so a token's row is the same whether the token is decoded
 * alone or inside a batch (a verify round reproducing single-token decode bit
 * for bit: "Fast single-box DeepSeek v4.1 Flash runtime", "Dependency order
 * and swarm split" and "Document map").  For one token the routing runs
 * inside the first kernel and the layer is three kernels (route + gate/up,
 * down, the fixed-order combine); larger T runs the four steps with their
 * intermediates in the workspace.
 *   arguments as moe_decode_layer;
 *   ws: moe_decode_layer_invariant_workspace_bytes(T, k, E, hidden, inter)
 *       bytes, 256-byte aligned; contents on entry do not matter
 * 1 <= T <= MOE_DECODE_MAX_TOKENS. */
MOE_FP4_API size_t moe_decode_layer_invariant_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t hidden,
                                                              int32_t inter);
MOE_FP4_API moe_status moe_decode_layer_invariant(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                                  int32_t k, const int32_t* expert_to_slot,
                                                  const moe_fp4_experts* w, const uint16_t* residual_bf16,
                                                  moe_out_dtype od, void* out, int32_t* topk_ids, float* topk_w,
                                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_decode_layer_noalloc -- moe_decode_layer for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments and the same results
 * bit for bit, without a workspace argument.  The workspace is instead a
 * static device array of the library, MOE_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on a GPU until the process ends; the call itself
 * allocates and frees nothing.  Its device address is looked up on the first
 * call on each GPU (with that GPU current), which should therefore happen
 * outside graph capture.  A call whose moe_decode_layer_workspace_bytes
 * exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE (one token at
 * the 5120 x 2304 shape takes 74 KB, 16 tokens 3.8 MB).  Nothing in the
 * array needs to start at zero.  All calls on one GPU share its array, so
 * calls that may overlap in time on one GPU (different streams, threads) race
 * on it and must be serialised by the caller; calls in stream order do not.
 * Unlike the other calls it keeps one piece of global state, the per-GPU
 * address of the array. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
MOE_FP4_API moe_status moe_decode_layer_noalloc(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                                int32_t k, const int32_t* expert_to_slot,
                                                const moe_fp4_experts* w, const uint16_t* residual_bf16,
                                                moe_out_dtype od, void* out, int32_t* topk_ids, float* topk_w,
                                                hipStream_t stream);

/* moe_decode_layer_gateup, moe_decode_layer_down -- the two halves of
 * moe_decode_layer with the same arguments: gateup routes (writing topk_ids,
 * topk_w and the routing state in ws) and runs the gate/up + SwiGLU weight
 * stream (h into ws); down runs the down-projection stream and the combine
 * into out.  gateup then down on one stream, with the same workspace, is
 * exactly moe_decode_layer.  They let a caller time or schedule the two
 * weight streams apart. */
MOE_FP4_API moe_status moe_decode_layer_gateup(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                               int32_t k, const int32_t* expert_to_slot,
                                               const moe_fp4_experts* w, const uint16_t* residual_bf16,
                                               moe_out_dtype od, void* out, int32_t* topk_ids, float* topk_w,
                                               void* ws, size_t ws_bytes, hipStream_t stream);
MOE_FP4_API moe_status moe_decode_layer_down(const float* logits, const uint16_t* x_bf16, int32_t T, int32_t E,
                                             int32_t k, const int32_t* expert_to_slot,
                                             const moe_fp4_experts* w, const uint16_t* residual_bf16,
                                             moe_out_dtype od, void* out, int32_t* topk_ids, float* topk_w,
                                             void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_decode_layer_rmsnorm -- one layer of a chained decode: the weightless
 * RMS norm of the bf16 residual rows x (exactly moe_rmsnorm_bf16 with eps),
 * then moe_decode_layer on the normalised rows with x itself as the
 * residual: out = x + sum_j w_j * FFN_j(rmsnorm(x)).  Bit-identical to
 * moe_rmsnorm_bf16 followed by moe_decode_layer: the harness layer of the
 * chained decode (the norm is the weightless one of moe_rmsnorm_bf16).  For
 * one token at the one-token shapes of moe_decode_layer the norm runs inside
 * its first kernel, which saves the norm kernel and its launch.
 *   arguments as moe_decode_layer; eps >= 0 (else MOE_ERR_SHAPE)
 *   ws: moe_decode_layer_rmsnorm_workspace_bytes(T, k, E, hidden, inter)
 *       bytes, 256-byte aligned; contents on entry do not matter
 * ------------------------------------------------------------------------- */
MOE_FP4_API size_t moe_decode_layer_rmsnorm_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t hidden,
                                                            int32_t inter);
MOE_FP4_API moe_status moe_decode_layer_rmsnorm(const float* logits, const uint16_t* x_bf16, float eps, int32_t T,
                                                int32_t E, int32_t k, const int32_t* expert_to_slot,
                                                const moe_fp4_experts* w, moe_out_dtype od, void* out,
                                                int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                                                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_ffn_fp4_prefill -- expert FFN of the prefill path on block-scaled MFMA.
 * Same contract as moe_ffn_fp4_decode except for the activation arithmetic,
 * which follows the activation-quantisation switch of the DGX Spark page
 * ("Reproduce the checks"; prefill and decode are separate arithmetic paths,
 * "Fast single-box DeepSeek v4.1 Flash runtime", "Conventions"): with
 * MOE_ACT_MXFP6_E2M3, x is quantised to MXFP6 (e2m3 codes, one UE8M0 scale
 * per 32 along hidden) before gate/up, and h (fp32) to MXFP6 along inter
 * before down.  Block exponent X = floor(log2 amax) - 2, plus 1 when the
 * significand of amax exceeds 1.875 (never saturates), clamped to
 * [-127, 127]; elements are rounded to nearest even.  Both GEMMs run on
 * gfx950 V_MFMA_SCALE_F32_32X32X64_F8F6F4 with e2m3 x e2m1 operands, whose
 * 32-term block sums are exact, accumulated in fp32.
 *   ws: at least moe_ffn_fp4_prefill_workspace_bytes(T, k, hidden, inter)
 *       bytes, 256-byte aligned
 *   the scale arrays of w must be 4-byte aligned on this path
 * T >= 1, T*k <= 2^22; the MXFP6 activations (x once per routed row, in
 * bucket order, and h) must each stay under 2 GiB (T*k*hidden*3/4 < 2^31 and
 * T*k*inter*3/4 < 2^31), else MOE_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
MOE_FP4_API size_t moe_ffn_fp4_prefill_workspace_bytes(int32_t T, int32_t k, int32_t hidden,
                                                       int32_t inter);
MOE_FP4_API moe_status moe_ffn_fp4_prefill(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                           const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                           const int32_t* expert_offsets,
                                           const int32_t* sorted_pair, moe_act_fmt act,
                                           float* y_pair, void* ws, size_t ws_bytes,
                                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_prefill_pack_weights, moe_ffn_fp4_prefill_packed -- moe_ffn_fp4_prefill
 * with its tiled GEMMs reading a second copy of the experts laid out in the
 * block-scaled MFMA's operand order.  Prefill re-reads each touched expert
 * once per tile of its tokens and is bound by how fast the weights reach the
 * matrix cores ("DeepSeek V4.1 Flash Q4 / 27 September 2026", "30 September
 * follow-up: prefill"); the copy is made once, when the experts are loaded.
 * Layout of the copy: for each slot, the gate, up and down matrices in turn
 * (gate and up: inter rows of hidden; down: hidden rows of inter), each as
 * blocks of 32 rows x 256 K elements, ordered by row block then K; a block is
 * 4 K-steps x 64 lanes x 16 code bytes (lane l: row l % 32, code bytes
 * 16 (l / 32) .. +15 of the K-step's 32 bytes of that row), then 64 lanes x
 * 4 scale bytes (byte S of lane l: the UE8M0 byte of the row's 32-block
 * 8 j + 2 S + l / 32, j the block's index along K).  Past K (inter % 256 ==
 * 128) codes and scales are zero.
 *   moe_prefill_packed_bytes(num_slots, hidden, inter): bytes of the copy
 *     (0 for an unsupported shape: hidden % 256 or inter % 128 nonzero)
 *   moe_prefill_pack_weights: writes the copy of every slot of w into
 *     packed (device, 256-byte aligned, packed_bytes at least the size above;
 *     MOE_ERR_WORKSPACE otherwise); asynchronous on stream
 *   moe_ffn_fp4_prefill_packed: arguments as moe_ffn_fp4_prefill, plus the
 *     copy of the same w.  The result is bit-identical to moe_ffn_fp4_prefill:
 *     the same MFMAs in the same order, only the weights' path differs.  Both
 *     the tiled GEMMs and the small-bucket kernels read the copy; w gives the
 *     shape and the slot count.  A copy that does not match w gives wrong
 *     results; a NULL or short copy with T >= 1 is MOE_ERR_NULL /
 *     MOE_ERR_WORKSPACE.
 * ------------------------------------------------------------------------- */
MOE_FP4_API size_t moe_prefill_packed_bytes(int32_t num_slots, int32_t hidden, int32_t inter);
MOE_FP4_API moe_status moe_prefill_pack_weights(const moe_fp4_experts* w, void* packed, size_t packed_bytes,
                                                hipStream_t stream);
MOE_FP4_API moe_status moe_ffn_fp4_prefill_packed(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                  const moe_fp4_experts* w, const void* packed,
                                                  size_t packed_bytes, const int32_t* expert_to_slot,
                                                  const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                  moe_act_fmt act, float* y_pair, void* ws, size_t ws_bytes,
                                                  hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_ffn_fp4_decode_subset, moe_ffn_fp4_prefill_subset -- the expert FFN
 * over a subset of the experts: the two-wave routed MoE of the M5 Max page
 * ("DeepSeek V4.1 Flash Q4 / 27 September 2026", "30 September follow-up:
 * prefill"), which computes the experts already on hand first and the rest
 * once they arrive.  Splitting the experts this way changes no bit of the
 * result, because each (token, slot) row is produced by exactly one call and
 * the rows are added together afterwards, in a fixed order, by moe_combine.
 *   run_mask [E] uint8 on the device: nonzero = run this expert's bucket now
 *   other arguments: as moe_ffn_fp4_decode / moe_ffn_fp4_prefill
 * Rows of the buckets whose mask byte is 0 are not written (their y_pair
 * rows keep whatever they held); every other row is exactly what the call
 * without a mask writes.  So calls whose masks cover each expert once, on
 * one stream (with one workspace, or one each), leave y_pair bit-identical
 * to one call over all experts, and each expert's weights are read by one
 * of them only.  A NULL run_mask with T >= 1 is MOE_ERR_NULL.
 * ------------------------------------------------------------------------- */
MOE_FP4_API moe_status moe_ffn_fp4_decode_subset(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                 const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                 const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                 const uint8_t* run_mask, float* y_pair, void* ws,
                                                 size_t ws_bytes, hipStream_t stream);
MOE_FP4_API moe_status moe_ffn_fp4_prefill_subset(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                                  const moe_fp4_experts* w, const int32_t* expert_to_slot,
                                                  const int32_t* expert_offsets, const int32_t* sorted_pair,
                                                  const uint8_t* run_mask, moe_act_fmt act, float* y_pair,
                                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_ffn_cb3_decode -- the decode expert FFN over a second expert codec, the
 * 3-bit per-row codebook in which the DGX Spark page stores the experts it
 * keeps routable, derived from the checkpoint's FP4 experts ("The
 * numbers").  The page fixes nothing more; the format
 * read here: every output row has a codebook of 8 bf16 values, and each
 * weight is a 3-bit index into its row's codebook, 8 indices per 3 bytes
 * (index i of a group in bits 3i..3i+2 of the little-endian 24-bit word).
 * W[n][c] = codebook[n][index[n][c]]; everything else -- buckets, arithmetic
 * (x bf16, fp32 sums, h fp32), y_pair, workspace -- is moe_ffn_fp4_decode's.
 *   q_gate, q_up : [num_slots][inter][hidden*3/8] index bytes (4-byte aligned)
 *   q_down       : [num_slots][hidden][inter*3/8]
 *   cb_gate, cb_up : [num_slots][inter][8] bf16 bits (16-byte aligned)
 *   cb_down        : [num_slots][hidden][8]
 * hidden % 256 == 0 and <= 6144, inter % 128 == 0 and <= 4096 (else
 * MOE_ERR_SHAPE / MOE_ERR_UNSUPPORTED); 1 <= T <= MOE_DECODE_MAX_TOKENS.
 * The encoder (packing FP4 experts into codebooks) is not part of the library.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t num_slots, hidden, inter;
  const uint8_t *q_gate, *q_up, *q_down;
  const uint16_t *cb_gate, *cb_up, *cb_down;
} moe_cb3_experts;

MOE_FP4_API size_t moe_ffn_cb3_decode_workspace_bytes(int32_t T, int32_t k, int32_t inter);
MOE_FP4_API moe_status moe_ffn_cb3_decode(const uint16_t* x_bf16, int32_t T, int32_t k, int32_t E,
                                          const moe_cb3_experts* w, const int32_t* expert_to_slot,
                                          const int32_t* expert_offsets, const int32_t* sorted_pair,
                                          float* y_pair, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_combine -- fixed-order weighted slot sum ("30 September follow-up").
 *   out[t] = sum_{j=0..k-1} topk_w[t][j] * y_pair[t*k+j]   (ascending j, fp32)
 *            + residual[t]                                 (if not NULL)
 * stored as bf16 (round to nearest even) or fp32.
 *   y_pair   [T*k][H] fp32 (16-byte aligned)
 *   topk_w   [T][k] fp32
 *   residual [T][H] bf16 bits or NULL
 *   out      [T][H] bf16 bits or fp32 (16-byte aligned; may not alias y_pair)
 * H % 8 == 0.
 * ------------------------------------------------------------------------- */
MOE_FP4_API moe_status moe_combine(const float* y_pair, const float* topk_w, int32_t T, int32_t k,
                                   int32_t H, const uint16_t* residual_bf16, moe_out_dtype od,
                                   void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_rmsnorm_bf16 -- weightless RMS norm of a bf16 residual stream,
 *   out[t] = bf16( x[t] / sqrt(mean(x[t]^2) + eps) )   (fp32 arithmetic).
 * Harness step of the chained multi-layer decode: the pages never restate
 * the architecture ("Fast single-box DeepSeek v4.1 Flash runtime", "Who this
 * is for"), and without a norm x <- x + MoE(x) overflows within a few layers.
 *   x, out [T][H] bf16 bits (16-byte aligned; out may alias x)
 * H % 8 == 0, H <= 65536.
 * ------------------------------------------------------------------------- */
MOE_FP4_API moe_status moe_rmsnorm_bf16(const uint16_t* x_bf16, int32_t T, int32_t H, float eps,
                                        uint16_t* out_bf16, hipStream_t stream);

/* Static description of a status code. */
MOE_FP4_API const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
