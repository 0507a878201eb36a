"""GPU parity of the decode path (router, bucketing, decode FFN, combine)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, W_TOL, GpuLayer, bf16_excess, rel_err, to_np

pytestmark = pytest.mark.gpu

DECODE_CASES = {
    "tiny": gi.CONFIGS["tiny"],
    # several row tiles, K-blocks that do not fill a wavefront, multi-token buckets
    "mid_zipf": gi.custom("mid_zipf", 1024, 384, 24, 4, 13, seed=21, zipf=1.1),
    # routable subset smaller than E, 3 slots per token
    "mid_resident": gi.custom("mid_resident", 768, 256, 40, 3, 9, seed=22, resident=12),
    "decode1": gi.CONFIGS["decode1"],
    "verify16": gi.CONFIGS["verify16"],
    # buckets of more than 16 rows (several row groups), 3 chunks of K in the down projection
    "groups40": gi.custom("groups40", 512, 384, 16, 4, 40, seed=23, zipf=1.1),
    # the largest decode batch: 256 tokens, buckets of up to 256 rows
    "batch256": gi.custom("batch256", 1024, 256, 8, 2, 256, seed=24),
    # fewer routable experts (3) than k (4): the last slot of every token takes a
    # non-routable expert with weight 0 and a zero row (multi-token and one-token kernels)
    "few_resident": gi.custom("few_resident", 512, 256, 16, 4, 9, seed=25, resident=3),
    "few_resident_1": gi.custom("few_resident_1", 1024, 256, 16, 4, 1, seed=26, resident=3),
}


def _oracle(gl: GpuLayer, mode="a16"):
    c = gl.cfg
    return o.moe_layer(gl.hi.x_bf16, gl.hi.logits[gl.layer], gl.weights.matrix, c.k, c.H, mode, gl.e2s_np)


def _check(name, r, ref, tol=REL_TOL):
    np.testing.assert_array_equal(to_np(r["ids"]), ref["ids"])
    np.testing.assert_array_equal(to_np(r["offsets"]), ref["offsets"])
    np.testing.assert_array_equal(to_np(r["sorted_pair"]), ref["sorted_pair"])
    np.testing.assert_array_equal(to_np(r["pair_to_row"]), ref["pair_to_row"])
    w = to_np(r["w"])
    assert np.max(np.abs(w - ref["w"])) <= W_TOL
    assert np.max(np.abs(w.sum(1) - 1.0)) <= W_TOL
    e_y = rel_err(to_np(r["y_pair"]), ref["y_pair"])
    e_32 = rel_err(to_np(r["out32"]), ref["out"])
    e_16 = bf16_excess(to_np(r["out16"]), ref["out"])
    print(f"[{name}] y_pair rel {e_y:.3e}  out fp32 rel {e_32:.3e}  out bf16 excess {e_16:.3e}", flush=True)
    assert e_y <= tol and e_32 <= tol and e_16 <= tol


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_layer_matches_oracle(name):
    print(f"case {name}", flush=True)
    gl = GpuLayer(DECODE_CASES[name])
    r = gl.run("decode")
    _check(name, r, _oracle(gl))


def test_decode_rotated_logits_full_size():
    """Several independent logit sets at the full decode shape (8 different experts each)."""
    cfg = gi.CONFIGS["decode1"]
    gl = GpuLayer(cfg)
    sets = gi.logit_sets(cfg, gl.hi.bias, 3)
    for i in range(3):
        logits = torch.from_numpy(sets[i]).cuda()
        r = gl.run("decode", logits=logits)
        ref = o.moe_layer(gl.hi.x_bf16, sets[i], gl.weights.matrix, cfg.k, cfg.H)
        _check(f"decode1/set{i}", r, ref)
        gl.weights.drop()


def test_decode_deterministic_and_batch_consistent():
    """Byte-identical reruns; a token's rows alone (the one-token kernels: VALU dot
    products in fp32) and inside the 16-token batch (the multi-token kernels: bf16
    MFMA with h as bf16 hi + lo) agree to 1e-5 of max|y|.  The two paths round
    differently, so they are not bit-identical: against the fp64 oracle the MFMA
    path measures <= 3.5e-6 and the one-token path <= 2e-7 of max|y| on every
    decode case, and 1e-5 leaves a margin of about three over their sum."""
    cfg = gi.CONFIGS["verify16"]
    gl = GpuLayer(cfg)
    a, b = gl.run("decode"), gl.run("decode")
    for key in ("y_pair", "out32", "out16", "w"):
        assert torch.equal(a[key], b[key]), key
    import fp4_routed_expert_mxfp4_amd as m
    for t in (0, 7, 15):
        ids, w = m.moe_route(gl.logits[t:t + 1].contiguous(), cfg.k)
        off, sp, _ = m.moe_permute(ids, cfg.E)
        y1 = m.moe_ffn_fp4_decode(gl.x[t:t + 1].contiguous(), cfg.k, cfg.E, gl.store, None, off, sp)
        torch.cuda.synchronize()
        ref = a["y_pair"][t * cfg.k:(t + 1) * cfg.k]
        e = rel_err(to_np(y1), to_np(ref).astype(np.float64))
        print(f"token {t}: alone vs in the batch {e:.2e}", flush=True)
        assert e <= 1e-5, t


def test_multi_token_batch_invariant_bit_exact():
    """With two or more tokens every row is one MFMA dot-product chain over the same
    K order, and the workgroup's K quarters are added in a fixed order: a token's
    y_pair rows are bit-identical whichever other tokens share its batch."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["verify16"]
    gl = GpuLayer(cfg)
    full = gl.run("decode")["y_pair"]
    k = cfg.k
    for sel in ([0, 1], [15, 3], list(range(8)), [5, 9, 12, 2, 14]):
        idx = torch.tensor(sel, device="cuda")
        ids, w = m.moe_route(gl.logits[idx].contiguous(), k)
        off, sp, _ = m.moe_permute(ids, cfg.E)
        y = m.moe_ffn_fp4_decode(gl.x[idx].contiguous(), k, cfg.E, gl.store, None, off, sp)
        torch.cuda.synchronize()
        for i, t in enumerate(sel):
            assert torch.equal(y[i * k:(i + 1) * k], full[t * k:(t + 1) * k]), (sel, t)


def test_invariant_decode_one_token_equals_batch_row():
    """moe_ffn_fp4_decode_invariant: each of the 16 verify tokens decoded alone gives
    the same y_pair rows, and the same combined output bits, as inside the
    16-token batch; one full-size token stays within the oracle tolerance."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["verify16"]
    gl = GpuLayer(cfg)
    r = gl.run("decode")
    k = cfg.k
    for t in range(cfg.T):
        ids, w = m.moe_route(gl.logits[t:t + 1].contiguous(), k)
        off, sp, _ = m.moe_permute(ids, cfg.E)
        y = m.moe_ffn_fp4_decode_invariant(gl.x[t:t + 1].contiguous(), k, cfg.E, gl.store, None, off, sp)
        out = m.moe_combine(y, w, None, m.MOE_OUT_BF16)
        torch.cuda.synchronize()
        assert torch.equal(y, r["y_pair"][t * k:(t + 1) * k]), t
        assert torch.equal(out.view(torch.int16), r["out16"][t:t + 1].view(torch.int16)), t
    c1 = gi.CONFIGS["decode1"]
    g1 = GpuLayer(c1)
    ids, w = m.moe_route(g1.logits, c1.k)
    off, sp, _ = m.moe_permute(ids, c1.E)
    y = m.moe_ffn_fp4_decode_invariant(g1.x, c1.k, c1.E, g1.store, None, off, sp)
    out = m.moe_combine(y, w, None, m.MOE_OUT_F32)
    torch.cuda.synchronize()
    ref = o.moe_layer(g1.hi.x_bf16, g1.hi.logits[0], g1.weights.matrix, c1.k, c1.H, "a16", None)
    e = rel_err(to_np(out), ref["out"])
    print(f"[decode1, invariant arithmetic] out fp32 rel {e:.3e}", flush=True)
    assert e <= REL_TOL


def test_integer_exact_case_bit_identical():
    """Weights +-1 and x = 1 keep every partial sum an integer below 2^24, and
    g >= 40 makes silu(g) == g in fp32 and fp64: the result must be exact."""
    import fp4_routed_expert_mxfp4_amd as m
    H, I, E, k, T = 256, 128, 4, 2, 3
    rng = np.random.default_rng(77)

    def codes(rows, K, p_plus):
        nib = np.where(rng.random((rows, K)) < p_plus, 0x2, 0xA).astype(np.uint8)
        return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)

    mats = {}
    for e in range(E):
        mats[(e, 0)] = (codes(I, H, 0.9), np.full((I, H // 32), 127, np.uint8))
        mats[(e, 1)] = (codes(I, H, 0.5), np.full((I, H // 32), 127, np.uint8))
        mats[(e, 2)] = (codes(H, I, 0.5), np.full((H, I // 32), 127, np.uint8))
    dev = torch.device("cuda")

    def stack(mi, part):
        return torch.from_numpy(np.stack([mats[(e, mi)][part] for e in range(E)])).to(dev)

    store = m.ExpertStore(stack(0, 0), stack(0, 1), stack(1, 0), stack(1, 1), stack(2, 0), stack(2, 1))
    x_np = gi.f32_to_bf16_bits(np.ones((T, H), np.float32))
    logits_np = rng.standard_normal((T, E)).astype(np.float32)
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    ids, w = m.moe_route(torch.from_numpy(logits_np).to(dev), k)
    off, sp, _ = m.moe_permute(ids, E)
    y = m.moe_ffn_fp4_decode(x, k, E, store, None, off, sp)
    torch.cuda.synchronize()
    ref_ids, _ = o.route(logits_np, k)
    ref_y = o.ffn(x_np, ref_ids, lambda e, mi: mats[(e, mi)], H)
    assert np.all(np.abs(ref_y) < 2 ** 24) and np.all(ref_y == np.round(ref_y))
    np.testing.assert_array_equal(to_np(y).astype(np.float64), ref_y)


def test_combine_and_rmsnorm_match_oracle():
    import fp4_routed_expert_mxfp4_amd as m
    rng = np.random.default_rng(5)
    T, k, H = 37, 8, 1280
    y = (rng.standard_normal((T * k, H)) * 1e5).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    res = gi.f32_to_bf16_bits((rng.standard_normal((T, H)) * 1e4).astype(np.float32))
    dev = torch.device("cuda")
    yt, wt = torch.from_numpy(y).to(dev), torch.from_numpy(w).to(dev)
    rt = torch.from_numpy(res.view(np.int16)).to(dev).view(torch.bfloat16)
    for residual in (None, rt):
        ref = o.combine(y.astype(np.float64), w.astype(np.float64), None if residual is None else res)
        o32 = to_np(m.moe_combine(yt, wt, residual, m.MOE_OUT_F32))
        o16 = to_np(m.moe_combine(yt, wt, residual, m.MOE_OUT_BF16))
        assert rel_err(o32, ref) <= 1e-6
        # the bf16 store is the RNE of the fp32 result
        np.testing.assert_array_equal(o16, gi.f32_to_bf16_bits(o32))
        assert bf16_excess(o16, ref) <= 1e-6
    xr = gi.f32_to_bf16_bits((rng.standard_normal((T, H)) * 3e5).astype(np.float32))
    xt = torch.from_numpy(xr.view(np.int16)).to(dev).view(torch.bfloat16)
    n = to_np(m.moe_rmsnorm_bf16(xt))
    ref = o.bf16_bits_to_f64(xr)
    ref = ref / np.sqrt(np.mean(ref * ref, axis=1, keepdims=True) + 1e-6)
    assert bf16_excess(n, ref) <= 1e-6
    ref_bits = o.rmsnorm_bf16(xr)
    # fp32 vs fp64 may round a handful of elements the other way; none by more than one ulp
    diff = np.abs(n.astype(np.int32) - ref_bits.astype(np.int32))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= T * H // 1000 + 1


def test_route_permute_prefill_shape_bit_exact():
    """Routing and bucketing of the 4096-token prefill chunk: bit-identical."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["prefill4096"]
    hi = gi.host_inputs(cfg)
    logits = torch.from_numpy(hi.logits[0]).cuda()
    ids, w = m.moe_route(logits, cfg.k)
    off, sp, p2r = m.moe_permute(ids, cfg.E)
    torch.cuda.synchronize()
    ref_ids, ref_w = o.route(hi.logits[0], cfg.k)
    np.testing.assert_array_equal(to_np(ids), ref_ids)
    assert np.max(np.abs(to_np(w) - ref_w)) <= W_TOL
    ref_off, ref_sp, ref_p2r = o.permute(ref_ids, cfg.E)
    np.testing.assert_array_equal(to_np(off), ref_off)
    np.testing.assert_array_equal(to_np(sp), ref_sp)
    np.testing.assert_array_equal(to_np(p2r), ref_p2r)
    counts = np.diff(ref_off)
    print(f"prefill4096 routing: {np.count_nonzero(counts)} experts touched, top bucket {counts.max()}")


def test_route_masked_and_edge_cases():
    import fp4_routed_expert_mxfp4_amd as m
    dev = torch.device("cuda")
    # ties, -0/+0, masked experts, k = E of the routable set, E not a multiple of 64, E = 1024
    rng = np.random.default_rng(8)
    for T, E, k, frac in [(5, 7, 3, 0.6), (33, 100, 8, 0.5), (3, 1024, 16, 0.3), (2, 64, 1, 1.0)]:
        logits = np.round(rng.standard_normal((T, E)) * 2).astype(np.float32)   # many ties
        logits[0, 0] = -0.0
        e2s = np.where(rng.random(E) < frac, 0, -1).astype(np.int32)
        e2s[rng.choice(E, k, replace=False)] = 0
        ids, w = m.moe_route(torch.from_numpy(logits).to(dev), k, torch.from_numpy(e2s).to(dev))
        ref_ids, ref_w = o.route(logits, k, e2s)
        np.testing.assert_array_equal(to_np(ids), ref_ids)
        assert np.max(np.abs(to_np(w) - ref_w)) <= W_TOL
        off, sp, p2r = m.moe_permute(ids, E)
        ref = o.permute(ref_ids, E)
        for a, b in zip((off, sp, p2r), ref):
            np.testing.assert_array_equal(to_np(a), b)


def test_route_all_ties_and_fewer_routable():
    """Every logit equal (each pick is decided by the lower expert index), and
    fewer routable experts than k: the routable ones come first in rank order
    with their softmax weights, then the best non-routable ones with weight 0."""
    import fp4_routed_expert_mxfp4_amd as m
    dev = torch.device("cuda")
    rng = np.random.default_rng(19)
    for E, k in [(384, 8), (1024, 16), (70, 6)]:
        logits = np.full((3, E), 0.75, np.float32)
        logits[1] = np.round(rng.standard_normal(E)).astype(np.float32)  # a few distinct values, many ties
        ids, w = m.moe_route(torch.from_numpy(logits).to(dev), k)
        ref_ids, ref_w = o.route(logits, k)
        np.testing.assert_array_equal(to_np(ids), ref_ids)
        assert np.max(np.abs(to_np(w) - ref_w)) <= W_TOL
        np.testing.assert_array_equal(to_np(ids)[0], np.arange(k))
    for E, k, n_rout in [(40, 8, 5), (384, 8, 0), (1024, 16, 15)]:
        logits = rng.standard_normal((4, E)).astype(np.float32)
        e2s = np.full(E, -1, np.int32)
        rout = np.sort(rng.choice(E, n_rout, replace=False))
        e2s[rout] = np.arange(n_rout, dtype=np.int32)
        ids, w = m.moe_route(torch.from_numpy(logits).to(dev), k, torch.from_numpy(e2s).to(dev))
        ids, w = to_np(ids), to_np(w)
        ref_ids, ref_w = o.route(logits, k, e2s)  # the oracle's fill reading (R-ROUTE-FILL)
        np.testing.assert_array_equal(ids, ref_ids)
        assert np.max(np.abs(w - ref_w)) <= W_TOL
        assert np.all(w[:, n_rout:] == 0)


def test_permute_large_and_empty():
    import fp4_routed_expert_mxfp4_amd as m
    dev = torch.device("cuda")
    rng = np.random.default_rng(12)
    T, k, E = 20000, 8, 384
    # heavy skew: half the pairs on a few experts
    ids = np.stack([rng.choice(E, k, replace=False, p=None) for _ in range(T)]).astype(np.int32)
    ids[: T // 2, 0] = 3
    off, sp, p2r = m.moe_permute(torch.from_numpy(ids).to(dev), E)
    # the stable order is unique: compare with a sort by (expert, pair)
    flat = ids.reshape(-1)
    order = np.lexsort((np.arange(flat.size), flat))
    np.testing.assert_array_equal(to_np(sp), order)
    np.testing.assert_array_equal(to_np(off), np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    np.testing.assert_array_equal(to_np(p2r), inv)
    # empty batch: offsets all zero
    off0, _, _ = m.moe_permute(torch.empty((0, k), dtype=torch.int32, device=dev), E)
    assert not to_np(off0).any()


@pytest.mark.parametrize("H,I", [(1024, 256), (2048, 2304)])
def test_one_token_repeated_expert_ids(H, I):
    """One token whose ids repeat an expert ([e, e, f, e]): its bucket holds the
    token several times, and every one of those rows is written (the one-token
    kernels compute the row once and store it per pair).  y_pair is checked
    against the oracle on every row, after filling it with a sentinel."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.custom(f"repeat_{H}_{I}", H, I, 8, 4, 1, seed=27)
    print(f"case repeated ids H={H} I={I}", flush=True)
    gl = GpuLayer(cfg)
    ids = np.array([[5, 5, 2, 5]], np.int32)
    off, sp, _ = m.moe_permute(torch.from_numpy(ids).cuda(), cfg.E)
    for call in (m.moe_ffn_fp4_decode, m.moe_ffn_fp4_decode_invariant):
        y = torch.full((cfg.k, cfg.H), 777.0, dtype=torch.float32, device="cuda")
        call(gl.x, cfg.k, cfg.E, gl.store, None, off, sp, y_pair=y)
        torch.cuda.synchronize()
        y_ref = o.ffn(gl.hi.x_bf16, ids, gl.weights.matrix, cfg.H)
        e = rel_err(to_np(y), y_ref)
        print(f"[repeat {H}x{I} {call.__name__}] y_pair rel {e:.3e}", flush=True)
        assert e <= REL_TOL
        yn = to_np(y)
        assert np.array_equal(yn[0], yn[1]) and np.array_equal(yn[0], yn[3])
