"""Plain fp64 CPU oracle for the routed MoE FFN over MXFP4 experts.

TEST INFRASTRUCTURE ONLY.  This module defines what the GPU path must
compute and is used solely by the tests, the smoke check and the benchmark's
CPU-baseline leg.  The product path never imports it, and it shares no code
with the HIP kernels or their Python binding.

Sources.  The pages describe the system this path belongs to:
  [DS4]   "Fast single-box DeepSeek v4.1 Flash runtime" (ds4-recipe mirror):
          Conventions (prefill and decode are separate arithmetic paths, each
          judged against its own reference; fixed summation orders are
          reference-defining); How to use this recipe (keep a correct slow
          baseline as the oracle).
  [M5]    "DeepSeek V4.1 Flash Q4 / 27 September 2026" (argonautlabs): the
          30 September follow-up (each (token, slot) pair has one output row,
          produced once, and a separate pass adds a token's rows in a fixed
          order).
  [SPARK] "DeepSeek-V4.1-Flash on a single NVIDIA DGX Spark" (shadowgraph):
          intro (the checkpoint's own e2m1 experts), Why it is built this way
          (15,360 experts x 3 x 2304 x 5120 weights, FP4 + UE8M0 per 32),
          The numbers (a kept subset of experts stays routable), Reproduce the
          checks (engine checked against a pure-torch reference with
          activation quantisation on).
  [OCP]   OCP Microscaling Formats (MX) Specification v1.0: the e2m1, e2m3 and
          E8M0 element/scale encodings.
The pages print no formula for routing, SwiGLU or dequantisation; where they
are silent the reading taken is stated at the function (R-... tags).

Every floating-point step is fp64.  The only library primitives are numpy's
matrix product (each output element is a plain dot product), exp and sort.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# Formats  [OCP] section 5 (element types) and 5.4 (E8M0 scale)
# --------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of a 4-bit e2m1 code: bits s e1 e0 m, exponent bias 1, no inf/NaN.

    E > 0: (-1)^s * 2^(E-1) * (1 + m/2);  E == 0: (-1)^s * m/2 (subnormal).
    """
    if not 0 <= code < 16:
        raise ValueError("e2m1 code out of range")
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = (2.0 ** (e - 1)) * (1.0 + m / 2.0) if e > 0 else m / 2.0
    return -mag if s else mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def ue8m0_value(byte: int) -> float:
    """UE8M0 scale byte -> 2^(byte-127).  0xFF (NaN in [OCP]) is rejected."""
    if not 0 <= byte < 255:
        raise ValueError("UE8M0 byte 255 (NaN) or out of range")
    return math.ldexp(1.0, byte - 127)


def decode_codes(codes: np.ndarray) -> np.ndarray:
    """Packed e2m1 bytes [..][K/2] -> fp64 values [..][K].

    R-NIB: element 2c sits in the low nibble of byte c, element 2c+1 in the
    high nibble (the pages do not fix the nibble order).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    lo = E2M1_TABLE[codes & 0x0F]
    hi = E2M1_TABLE[codes >> 4]
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[n][c] = e2m1(code[n][c]) * 2^(scale[n][c // 32] - 127), exact in fp64.

    [SPARK] "Why it is built this way": FP4 weights with one UE8M0 scale per
    32 weights; a block covers 32 contiguous K-elements of one row.
    R-ORI: matrices are stored [out][in] with K (the reduction dim) contiguous.
    """
    scales = np.asarray(scales, dtype=np.uint8)
    if np.any(scales == 255):
        raise ValueError("UE8M0 byte 255 (NaN) in weights")
    v = decode_codes(codes)
    rows, K = v.shape[-2], v.shape[-1]
    if scales.shape[-1] * 32 != K:
        raise ValueError("scale count does not match K/32")
    mult = np.ldexp(1.0, scales.astype(np.int64) - 127)          # exact powers of two
    return (v.reshape(rows, K // 32, 32) * mult[..., None]).reshape(rows, K)


# --------------------------------------------------------------------------
# Router
# --------------------------------------------------------------------------


def route(logits: np.ndarray, k: int, expert_to_slot: np.ndarray | None = None):
    """Top-k routing with softmax over the selected k.

    Candidates: experts with expert_to_slot[e] >= 0 (all when the table is
    absent) -- [SPARK] "The numbers": only a kept subset of experts stays
    routable.  Order candidates by (logit descending, expert index ascending);
    slot j of the token holds rank j.  Weights are
    w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected.
    R-ROUTE: the pages give no scoring function; this plain reading uses the
    raw fp32 logits, ties go to the lower expert index, -0 == +0.
    R-ROUTE-FILL: the pages do not say what a token gets when fewer than k of
    its experts are routable.  Reading: the routable experts come first, in
    the order above, and the remaining slots take the non-routable experts in
    the same order with weight 0; the softmax runs over the routable slots
    only (all weights are 0 when none is routable).  Their rows then hold an
    expert with no stored weights, whose FFN rows are zero.
    Non-finite logits and k outside [1, E] are rejected.
    Returns ids int32 [T][k] and weights fp64 [T][k].
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not np.all(np.isfinite(logits)):
        raise ValueError("non-finite logit")
    if not 1 <= k <= E:
        raise ValueError("k must lie in [1, E]")
    routable = [e for e in range(E) if expert_to_slot is None or int(expert_to_slot[e]) >= 0]
    others = [e for e in range(E) if expert_to_slot is not None and int(expert_to_slot[e]) < 0]
    ids = np.empty((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        rank = lambda e: (-row[e], e)
        sel = (sorted(routable, key=rank) + sorted(others, key=rank))[:k]
        ids[t] = sel
        n = min(k, len(routable))              # the routable slots come first
        if n:
            l = np.array([row[e] for e in sel[:n]], dtype=np.float64)
            ex = np.exp(l - l[0])
            w[t, :n] = ex / ex.sum()
    return ids, w


def router_logits(x_bf16: np.ndarray, w_router_bf16: np.ndarray, bias=None) -> np.ndarray:
    """Router gate projection: logits[t][e] = sum_c x[t][c] * W_r[e][c] + bias[e].

    The router runs before expert selection and the experts' reads cannot
    start until it has ([M5] "30 September follow-up: prefill"; the split
    router of "4 October follow-up"), but no page gives its form or
    precision.  R-GATE: the
    plain linear gate of a routed MoE layer -- W_r holds one row per expert
    over the hidden size, in bf16 like the activations; bias (optional, one
    value per expert, given as float32) is added to the dot product.  Here it
    carries the per-expert popularity bias of the skewed synthetic routings.
    x and W_r arrive as bf16 bit patterns; every step is fp64.
    Returns fp64 [T][E].
    """
    x = bf16_bits_to_f64(x_bf16)
    w = bf16_bits_to_f64(w_router_bf16)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x [T][H] and W_r [E][H] must share H")
    out = x @ w.T
    if bias is not None:
        b = np.asarray(bias, dtype=np.float32).astype(np.float64)
        if b.shape != (w.shape[0],):
            raise ValueError("bias must hold one value per expert")
        out = out + b
    return out


def route_from_x(x_bf16, w_router_bf16, k: int, bias=None, expert_to_slot=None):
    """Gate projection, then top-k routing (route above).

    The logits are held as float32 (the router's input type), so the
    selection is taken on the fp64 logits rounded once to float32.
    Returns (logits fp64 [T][E], ids int32 [T][k], weights fp64 [T][k]).
    """
    l = router_logits(x_bf16, w_router_bf16, bias)
    ids, w = route(l.astype(np.float32), k, expert_to_slot)
    return l, ids, w


# --------------------------------------------------------------------------
# Token -> expert bucketing
# --------------------------------------------------------------------------


def permute(ids: np.ndarray, E: int):
    """Stable bucketing of the (token, slot) pairs by expert.

    Pair p = t*k + j.  counts[e] = #{p: ids[p] = e}; offsets = exclusive
    prefix sum with offsets[E] = T*k; sorted_pair lists all p ordered by
    (expert ascending, p ascending); pair_to_row is its inverse.  The
    (token, slot) rows are those of [M5] "30 September follow-up".
    """
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pair = np.array(sorted(range(flat.size), key=lambda p: (flat[p], p)), dtype=np.int32)
    pair_to_row = np.empty(flat.size, dtype=np.int32)
    pair_to_row[sorted_pair] = np.arange(flat.size, dtype=np.int32)
    return offsets, sorted_pair, pair_to_row


# --------------------------------------------------------------------------
# Activation encoding of the prefill path (R-ACT): MXFP6 E2M3
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e2m3_value(code: int) -> float:
    """[OCP] FP6 E2M3: bits s e1 e0 m2 m1 m0, exponent bias 1, no inf/NaN.

    E > 0: (-1)^s * 2^(E-1) * (1 + m/8);  E == 0: (-1)^s * m/8.  Max 7.5.
    """
    if not 0 <= code < 64:
        raise ValueError("e2m3 code out of range")
    s, e, m = code >> 5, (code >> 3) & 3, code & 7
    mag = (2.0 ** (e - 1)) * (1.0 + m / 8.0) if e > 0 else m / 8.0
    return -mag if s else mag


E2M3_TABLE = np.array([e2m3_value(c) for c in range(64)], dtype=np.float64)
E2M3_MAX = 7.5


def e2m3_encode(t: np.ndarray) -> np.ndarray:
    """Round t (already divided by the block scale) to the e2m3 grid, RNE.

    Binades [1,2), [2,4), [4,8) keep 3 mantissa bits; below 1 the step is 1/8.
    Magnitudes above 7.5 saturate to 7.5 (only reachable when the shared
    exponent was clamped at -127).  The sign bit is the sign of t.
    """
    t = np.asarray(t, dtype=np.float64)
    sign = np.where(np.signbit(t), 0x20, 0).astype(np.int64)
    a = np.abs(t)
    e = np.frexp(a)[1] - 1                                  # a in [2^e, 2^(e+1)) for a > 0
    quantum = np.ldexp(1.0, np.maximum(e - 3, -3))
    q = np.minimum(np.rint(a / quantum) * quantum, E2M3_MAX)  # rint rounds half to even
    qe = np.frexp(q)[1] - 1
    normal = q >= 1.0
    m_norm = np.where(normal, (np.ldexp(q, -np.where(normal, qe, 0)) - 1.0) * 8.0, 0.0)
    code_norm = ((qe + 1) << 3) + m_norm.astype(np.int64)
    code_sub = (q * 8.0).astype(np.int64)
    return (sign | np.where(normal, code_norm, code_sub)).astype(np.uint8)


def q6_rows(a: np.ndarray):
    """MXFP6 (e2m3) quantisation along the last axis in 32-blocks.  R-ACT.

    Per block: shared exponent X = floor(log2 amax) - 2, plus one when the
    significand of amax exceeds 1.875 -- the smallest power-of-two scale
    under which no element exceeds 7.5, so nothing saturates; X is clamped
    to [-127, 127]; scale byte = X + 127.  A block with amax == 0 gets scale
    byte 0 and all-zero codes.  Elements are v * 2^-X rounded to nearest
    even on the e2m3 grid.  [OCP] defines the encodings; the pages only show
    an activation-quantisation switch ([SPARK] "Reproduce the checks").
    Returns (codes uint8 [rows][K], scale bytes uint8 [rows][K/32]).
    """
    a = np.asarray(a, dtype=np.float64)
    rows, K = a.shape
    blocks = a.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(blocks), axis=2)
    frac, ex = np.frexp(amax)                  # amax = frac * 2^ex, frac in [0.5, 1)
    E, M = ex - 1, 2.0 * frac                  # amax = M * 2^E, M in [1, 2)
    X = np.clip(E - 2 + (M > 1.875), -127, 127)
    zero = amax == 0.0
    X = np.where(zero, -127, X)
    codes = e2m3_encode(np.ldexp(blocks, -X[..., None]))
    codes[zero] = 0
    return codes.reshape(rows, K), (X + 127).astype(np.uint8)


def q6_block(v: np.ndarray):
    """Q6 of a single 32-element block: (codes uint8[32], scale byte)."""
    c, s = q6_rows(np.asarray(v, dtype=np.float64).reshape(1, 32))
    return c[0], int(s[0, 0])


def q6_dequant(codes: np.ndarray, sb: np.ndarray) -> np.ndarray:
    rows, K = codes.shape
    v = E2M3_TABLE[codes].reshape(rows, K // 32, 32)
    return (v * np.ldexp(1.0, sb.astype(np.int64) - 127)[..., None]).reshape(rows, K)


def round_f32(a: np.ndarray) -> np.ndarray:
    """Round fp64 to the nearest float32 (RNE) and return it as fp64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Expert FFN
# --------------------------------------------------------------------------


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u = g * u / (1 + exp(-g)).  R-SWI: no clamp, no biases."""
    with np.errstate(over="ignore"):
        return g * u / (1.0 + np.exp(-g))


def expert_ffn(x: np.ndarray, weights, expert: int, mode: str = "a16") -> np.ndarray:
    """y = W_down . swiglu(W_gate . x, W_up . x) for the rows of x (fp64 [m][H]).

    weights(expert, matrix) -> (codes, scales) with matrix 0 gate, 1 up,
    2 down.  mode "a16": x as given, no intermediate rounding (the decode
    reference).  mode "a6" (R-ACT, the prefill reference): x is replaced by
    Q6(x) before gate/up, and h by Q6(h) before down, h being rounded to
    float32 first so the quantiser decides on the same precision the kernel
    holds h in.  Prefill and decode are separate arithmetic paths judged
    against their own references ([DS4] "Conventions").
    """
    wg = dequant(*weights(expert, 0))
    wu = dequant(*weights(expert, 1))
    wd = dequant(*weights(expert, 2))
    if mode == "a6":
        x = q6_dequant(*q6_rows(x))
    elif mode != "a16":
        raise ValueError(mode)
    h = swiglu(x @ wg.T, x @ wu.T)
    if mode == "a6":
        h = q6_dequant(*q6_rows(round_f32(h)))
    return h @ wd.T


def ffn(x_bf16: np.ndarray, ids: np.ndarray, weights, H: int, mode: str = "a16",
        expert_to_slot: np.ndarray | None = None) -> np.ndarray:
    """y_pair fp64 [T*k][H]: row p = t*k + j is expert ids[t][j] applied to x_t.

    With an expert_to_slot table, an expert without a slot (entry < 0) has no
    stored weights and its rows are zero (R-ROUTE-FILL: such experts fill the
    slots of a token with fewer than k routable experts, at weight 0).
    """
    x = bf16_bits_to_f64(x_bf16)
    T, k = ids.shape
    y = np.zeros((T * k, H), dtype=np.float64)
    flat = ids.reshape(-1)
    for e in sorted(set(int(v) for v in flat)):
        if expert_to_slot is not None and int(expert_to_slot[e]) < 0:
            continue
        pairs = np.nonzero(flat == e)[0]
        y[pairs] = expert_ffn(x[pairs // k], weights, e, mode)
    return y


# --------------------------------------------------------------------------
# Second expert codec: 3-bit per-row codebook (R-CB3)
# --------------------------------------------------------------------------


def cb3_indices(qbytes: np.ndarray, K: int) -> np.ndarray:
    """Packed 3-bit indices [rows][3K/8] bytes -> int [rows][K].

    R-CB3: the DGX Spark page ("The numbers") stores the experts it keeps
    routable with 3 bits per weight and a codebook per row, derived from the
    checkpoint's FP4 experts, and gives no further detail.  Reading: every group of 8 consecutive indices of a row
    is one 24-bit little-endian word in 3 bytes; index i of the group sits in
    bits 3i..3i+2.
    """
    q = np.asarray(qbytes, dtype=np.uint8)
    rows = q.shape[0]
    if K % 8 or q.shape[1] * 8 != K * 3:
        raise ValueError("cb3 rows hold 3 bytes per 8 weights")
    b = q.reshape(rows, K // 8, 3).astype(np.uint32)
    word = b[..., 0] | (b[..., 1] << np.uint32(8)) | (b[..., 2] << np.uint32(16))
    idx = (word[..., None] >> (np.uint32(3) * np.arange(8, dtype=np.uint32))) & np.uint32(7)
    return idx.reshape(rows, K).astype(np.int64)


def cb3_dequant(qbytes: np.ndarray, codebook_bf16: np.ndarray) -> np.ndarray:
    """W[n][c] = codebook[n][index[n][c]] in fp64.  R-CB3: each output row has
    its own codebook of 8 values, held as bf16 (a value of the FP4 checkpoint,
    an e2m1 code times a power of two, is exact in bf16)."""
    cb = bf16_bits_to_f64(np.asarray(codebook_bf16, dtype=np.uint16))
    if cb.ndim != 2 or cb.shape[1] != 8:
        raise ValueError("one codebook of 8 entries per row")
    K = np.asarray(qbytes).shape[1] * 8 // 3
    idx = cb3_indices(qbytes, K)
    return np.take_along_axis(cb, idx, axis=1)


def ffn_cb3(x_bf16: np.ndarray, ids: np.ndarray, weights, H: int) -> np.ndarray:
    """y_pair fp64 [T*k][H] for cb3 experts: as ffn (mode "a16", the decode
    reference) with W from cb3_dequant.  weights(expert, matrix) -> (index
    bytes, codebook) with matrix 0 gate, 1 up, 2 down."""
    x = bf16_bits_to_f64(x_bf16)
    T, k = ids.shape
    y = np.zeros((T * k, H), dtype=np.float64)
    flat = ids.reshape(-1)
    for e in sorted(set(int(v) for v in flat)):
        pairs = np.nonzero(flat == e)[0]
        wg = cb3_dequant(*weights(e, 0))
        wu = cb3_dequant(*weights(e, 1))
        wd = cb3_dequant(*weights(e, 2))
        xe = x[pairs // k]
        y[pairs] = swiglu(xe @ wg.T, xe @ wu.T) @ wd.T
    return y


# --------------------------------------------------------------------------
# Combine and bf16 store
# --------------------------------------------------------------------------


def combine(y_pair: np.ndarray, w: np.ndarray, residual_bf16: np.ndarray | None = None) -> np.ndarray:
    """out_t = sum_{j=0..k-1} w[t][j] * y[t*k+j] (ascending j) + residual_t.

    [M5] "30 September follow-up": the slot sum is its own fixed-order step
    over rows that were each written once.
    """
    T, k = w.shape
    out = np.zeros((T, y_pair.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y_pair[j::k]
    if residual_bf16 is not None:
        out += bf16_bits_to_f64(residual_bf16)
    return out


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns, round to nearest even, directly from fp64.

    bf16 keeps 8 significant bits; below 2^-126 the step is 2^-133; values
    past the largest finite bf16 become infinity.
    """
    a = np.asarray(a, dtype=np.float64)
    e = np.frexp(np.abs(a))[1] - 1
    quantum = np.ldexp(1.0, np.maximum(e - 7, -133))
    q = np.rint(a / quantum) * quantum
    q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, q), q)
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# Whole layer and the 40-layer chain
# --------------------------------------------------------------------------


def moe_layer(x_bf16, logits, weights, k, H, mode="a16", expert_to_slot=None, residual_bf16=None):
    """Router -> bucketing -> expert FFN -> fixed-order combine, all fp64."""
    E = logits.shape[1]
    ids, w = route(logits, k, expert_to_slot)
    offsets, sorted_pair, pair_to_row = permute(ids, E)
    y = ffn(x_bf16, ids, weights, H, mode, expert_to_slot)
    out = combine(y, w, residual_bf16)
    return dict(ids=ids, w=w, offsets=offsets, sorted_pair=sorted_pair,
                pair_to_row=pair_to_row, y_pair=y, out=out)


def rmsnorm_bf16(x_bf16: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """n = bf16(x / sqrt(mean(x^2) + eps)) per token, weightless.

    R-CHAIN: the pages never re-specify the architecture ([DS4] "Who this is
    for"); read literally, x <- x + MoE(x) overflows within a few layers, so
    each layer's MoE input is a weightless RMS norm of the residual stream.
    """
    x = bf16_bits_to_f64(x_bf16)
    r = np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return bf16_rne(x / r)


def chain_layer(x_bf16, logits, weights, k, H, expert_to_slot):
    """One chained decode layer: x' = bf16(x + MoE(rmsnorm(x)))."""
    n = rmsnorm_bf16(x_bf16)
    res = moe_layer(n, logits, weights, k, H, "a16", expert_to_slot, residual_bf16=x_bf16)
    res["norm"] = n
    res["x_next"] = bf16_rne(res["out"])
    return res
