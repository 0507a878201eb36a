"""moe_decode_layer (route + bucketing + decode FFN + combine in one call)
through the C ABI: bit-identical to the four separate calls, and within
tolerance of the fp64 oracle.  One-token shapes take the two-kernel fused
path; the others run the separate kernels inside the call."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, W_TOL, GpuLayer, bf16_excess, rel_err, to_np

pytestmark = pytest.mark.gpu


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def _layer(m, gl: GpuLayer, logits, residual, od):
    out, ids, w = m.moe_decode_layer(logits, gl.x, gl.cfg.k, gl.store, gl.e2s, residual, od)
    torch.cuda.synchronize()
    return out, ids, w


def _same_as_separate(m, gl: GpuLayer, logits=None, residual=None):
    """The one call against route -> permute -> decode -> combine, for both output types."""
    logits = gl.logits if logits is None else logits
    r = gl.run("decode", logits=logits, residual=residual)
    res = {}
    for od, key in ((m.MOE_OUT_F32, "out32"), (m.MOE_OUT_BF16, "out16")):
        out, ids, w = _layer(m, gl, logits, residual, od)
        assert torch.equal(ids, r["ids"])
        assert torch.equal(w, r["w"])
        assert torch.equal(out, r[key]), key
        res[key] = out
    # the two halves as separate calls through one workspace
    cfg = gl.cfg
    ws = torch.empty(max(m.decode_layer_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I), 256),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(r["out16"])
    ids = torch.empty_like(r["ids"])
    w = torch.empty_like(r["w"])
    for phase in (1, 2):
        m.moe_decode_layer(logits, gl.x, cfg.k, gl.store, gl.e2s, residual, m.MOE_OUT_BF16, out, ids, w, ws,
                           phase=phase)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out16"]) and torch.equal(ids, r["ids"]) and torch.equal(w, r["w"])
    return r, res


def test_fused_decode1_rotated_bit_identical_and_oracle():
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["decode1"]
    gl = GpuLayer(cfg)
    assert m.decode_layer_workspace_bytes(1, cfg.k, cfg.E, cfg.H, cfg.I) == 512 + cfg.k * cfg.I * 4
    sets = gi.logit_sets(cfg, gl.hi.bias, 3)
    rng = np.random.default_rng(41)
    res_np = gi.f32_to_bf16_bits((rng.standard_normal((1, cfg.H)) * 4e5).astype(np.float32))
    for i in range(3):
        print(f"decode1 logit set {i}", flush=True)
        logits = torch.from_numpy(sets[i]).cuda()
        residual = _bf16(res_np) if i == 1 else None
        r, got = _same_as_separate(m, gl, logits, residual)
        ref = o.moe_layer(gl.hi.x_bf16, sets[i], gl.weights.matrix, cfg.k, cfg.H)
        np.testing.assert_array_equal(to_np(r["ids"]), ref["ids"])
        assert np.max(np.abs(to_np(r["w"]) - ref["w"])) <= W_TOL
        ref_out = ref["out"] if residual is None else o.combine(ref["y_pair"], ref["w"], res_np)
        e32 = rel_err(to_np(got["out32"]), ref_out)
        e16 = bf16_excess(to_np(got["out16"]), ref_out)
        print(f"[decode1/set{i}{' +residual' if residual is not None else ''}] fp32 rel {e32:.3e} "
              f"bf16 excess {e16:.3e}", flush=True)
        assert e32 <= REL_TOL and e16 <= REL_TOL
        gl.weights.drop()


def test_fused_chain_layer_masked_routing():
    """A chain layer: 154 of 384 experts stored, routing masked to them, bf16 residual."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["chain40"]
    hi = gi.host_inputs(cfg)
    gl = GpuLayer(cfg, layer=7, hi=hi)
    rng = np.random.default_rng(7)
    res_np = gi.f32_to_bf16_bits((rng.standard_normal((1, cfg.H)) * 3e5).astype(np.float32))
    r, got = _same_as_separate(m, gl, residual=_bf16(res_np))
    ref_ids, ref_w = o.route(hi.logits[7], cfg.k, hi.expert_to_slot[7])
    np.testing.assert_array_equal(to_np(r["ids"]), ref_ids)
    y = o.ffn(hi.x_bf16, ref_ids, gl.weights.matrix, cfg.H)
    ref = o.combine(y, ref_w, res_np)
    e16 = bf16_excess(to_np(got["out16"]), ref)
    print(f"[chain40 layer 7] bf16 excess {e16:.3e}", flush=True)
    assert e16 <= REL_TOL


FUSED_SHAPES = {
    # inter = 256: only the 8-block tail of the down row (M = 0), k = 4, hidden of one 1024-block
    "h1024_i256": gi.custom("fl_a", 1024, 256, 16, 4, 1, seed=51),
    # inter = 2048: no tail, hidden 6144 (the largest fused shape), k = 1
    "h6144_i2048_k1": gi.custom("fl_b", 6144, 2048, 8, 1, 1, seed=52),
    # E not a multiple of 64 with a masked subset, k = 6
    "h2048_i2304_masked": gi.custom("fl_c", 2048, 2304, 70, 6, 1, seed=53, resident=20),
}


@pytest.mark.parametrize("name", list(FUSED_SHAPES))
def test_fused_shapes_bit_identical(name):
    import fp4_routed_expert_mxfp4_amd as m
    cfg = FUSED_SHAPES[name]
    print(f"case {name}", flush=True)
    gl = GpuLayer(cfg)
    assert m.decode_layer_workspace_bytes(1, cfg.k, cfg.E, cfg.H, cfg.I) == \
        512 + ((cfg.k * cfg.I * 4 + 255) // 256) * 256
    r, got = _same_as_separate(m, gl)
    ref = o.moe_layer(gl.hi.x_bf16, gl.hi.logits[0], gl.weights.matrix, cfg.k, cfg.H, "a16", gl.e2s_np)
    e32 = rel_err(to_np(got["out32"]), ref["out"])
    print(f"[{name}] fp32 rel {e32:.3e}", flush=True)
    assert e32 <= REL_TOL


FALLBACK = {
    "tiny": gi.CONFIGS["tiny"],                       # hidden 256: not a fused shape
    "verify16": gi.CONFIGS["verify16"],               # 16 tokens
    "mid_resident": gi.custom("fl_mid", 768, 256, 40, 3, 9, seed=22, resident=12),
}


@pytest.mark.parametrize("name", list(FALLBACK))
def test_unfused_shapes_bit_identical(name):
    import fp4_routed_expert_mxfp4_amd as m
    cfg = FALLBACK[name]
    print(f"case {name}", flush=True)
    gl = GpuLayer(cfg)
    ws = m.decode_layer_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I)
    assert ws >= cfg.T * cfg.k * (cfg.H + cfg.I) * 4
    rng = np.random.default_rng(3)
    res_np = gi.f32_to_bf16_bits((rng.standard_normal((cfg.T, cfg.H)) * 10).astype(np.float32))
    for residual in (None, _bf16(res_np)):
        _same_as_separate(m, gl, residual=residual)


def test_fused_graph_replays():
    """The fused layer captured in a HIP graph: every replay equals the eager call."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["decode1"]
    gl = GpuLayer(cfg)
    sets = [torch.from_numpy(a).cuda() for a in gi.logit_sets(cfg, gl.hi.bias, 2)]
    logits = sets[0].clone()
    out = torch.empty((1, cfg.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((1, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, cfg.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.decode_layer_workspace_bytes(1, cfg.k, cfg.E, cfg.H, cfg.I), dtype=torch.uint8,
                     device="cuda")
    eager = []
    for s in sets:
        logits.copy_(s)
        m.moe_decode_layer(logits, gl.x, cfg.k, gl.store, None, None, m.MOE_OUT_BF16, out, ids, w, ws)
        torch.cuda.synchronize()
        eager.append((out.clone(), ids.clone(), w.clone()))
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            m.moe_decode_layer(logits, gl.x, cfg.k, gl.store, None, None, m.MOE_OUT_BF16, out, ids, w, ws)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        i = rep % 2
        logits.copy_(sets[i])
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[i][0]) and torch.equal(ids, eager[i][1]) and torch.equal(w, eager[i][2]), rep


NORM_SHAPES = {
    "decode1": gi.CONFIGS["decode1"],                                  # the norm inside K1, hidden 5120
    "h6144_i2048_k1": FUSED_SHAPES["h6144_i2048_k1"],                  # the largest one-token hidden (6144)
    "h1024_i256": FUSED_SHAPES["h1024_i256"],
    "verify16": gi.CONFIGS["verify16"],                                # 16 rows: norm kernel + the layer
    "tiny": gi.CONFIGS["tiny"],
}


@pytest.mark.parametrize("name", list(NORM_SHAPES))
def test_rmsnorm_layer_bit_identical(name):
    """moe_decode_layer_rmsnorm against moe_rmsnorm_bf16 then moe_decode_layer with x as
    the residual: the same bits, for residual streams of chain-like magnitude."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = NORM_SHAPES[name]
    print(f"case {name}", flush=True)
    gl = GpuLayer(cfg)
    rng = np.random.default_rng(17)
    for scale in (3e5, 1.0):
        x_np = gi.f32_to_bf16_bits((rng.standard_normal((cfg.T, cfg.H)) * scale).astype(np.float32))
        x = _bf16(x_np)
        n = m.moe_rmsnorm_bf16(x, 1e-6)
        for od in (m.MOE_OUT_BF16, m.MOE_OUT_F32):
            ref, ids_r, w_r = m.moe_decode_layer(gl.logits, n, cfg.k, gl.store, gl.e2s, x, od)
            got, ids, w = m.moe_decode_layer_rmsnorm(gl.logits, x, cfg.k, gl.store, 1e-6, gl.e2s, od)
            torch.cuda.synchronize()
            assert torch.equal(ids, ids_r) and torch.equal(w, w_r)
            assert torch.equal(got, ref), (name, scale, od)


def test_rmsnorm_chain_layer_masked():
    """A chain layer (154 of 384 experts, masked routing) through the norm-folded call."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["chain40"]
    hi = gi.host_inputs(cfg)
    gl = GpuLayer(cfg, layer=11, hi=hi)
    rng = np.random.default_rng(11)
    x = _bf16(gi.f32_to_bf16_bits((rng.standard_normal((1, cfg.H)) * 3e5).astype(np.float32)))
    n = m.moe_rmsnorm_bf16(x, 1e-6)
    ref, ids_r, _ = m.moe_decode_layer(gl.logits, n, cfg.k, gl.store, gl.e2s, x, m.MOE_OUT_BF16)
    got, ids, _ = m.moe_decode_layer_rmsnorm(gl.logits, x, cfg.k, gl.store, 1e-6, gl.e2s, m.MOE_OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_r) and torch.equal(got, ref)
