"""The batch-invariant decode layer in one call (moe_decode_layer_invariant):
bit-identical to the four separate calls on the invariant arithmetic (route,
permute, moe_ffn_fp4_decode_invariant, combine), a token decoded alone equal
bit for bit to its row in a batch, and within the oracle tolerance."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, W_TOL, GpuLayer, bf16_excess, rel_err, to_np

pytestmark = pytest.mark.gpu

ONE_TOKEN = {
    "decode1": gi.CONFIGS["decode1"],
    "tiny": gi.CONFIGS["tiny"],
    # the routable subset of a chain layer (154 of 384 resident)
    "resident": gi.custom("resident", 1024, 256, 64, 8, 1, seed=41, resident=20),
    # fewer routable experts (3) than k (4): a weight-0 slot with a zero row
    "few_resident": gi.custom("few_resident", 1024, 256, 16, 4, 1, seed=42, resident=3),
    # 1024 experts (16 logits per lane in the router), k = 16, inter not a multiple of 256
    "wide": gi.custom("wide", 768, 384, 1024, 16, 1, seed=43),
}


def _four_calls(gl: GpuLayer, x, logits, residual, od):
    import fp4_routed_expert_mxfp4_amd as m
    c = gl.cfg
    ids, w = m.moe_route(logits, c.k, gl.e2s)
    off, sp, _ = m.moe_permute(ids, c.E)
    y = m.moe_ffn_fp4_decode_invariant(x, c.k, c.E, gl.store, gl.e2s, off, sp)
    out = m.moe_combine(y, w, residual, od)
    return out, ids, w


@pytest.mark.parametrize("name", list(ONE_TOKEN))
def test_invariant_layer_equals_four_calls(name):
    import fp4_routed_expert_mxfp4_amd as m
    cfg = ONE_TOKEN[name]
    gl = GpuLayer(cfg)
    res = (gl.x * 0.5).contiguous()
    for od, residual in ((m.MOE_OUT_BF16, None), (m.MOE_OUT_F32, res)):
        out, ids, w = m.moe_decode_layer_invariant(gl.logits, gl.x, cfg.k, gl.store, gl.e2s, residual, od)
        out4, ids4, w4 = _four_calls(gl, gl.x, gl.logits, residual, od)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids4) and torch.equal(w, w4), (name, od)
        assert torch.equal(out.view(torch.int32 if od == m.MOE_OUT_F32 else torch.int16),
                           out4.view(torch.int32 if od == m.MOE_OUT_F32 else torch.int16)), (name, od)
    # against the oracle: the routing exactly, the output within the tolerance
    out32, ids, w = m.moe_decode_layer_invariant(gl.logits, gl.x, cfg.k, gl.store, gl.e2s, None, m.MOE_OUT_F32)
    out16, _, _ = m.moe_decode_layer_invariant(gl.logits, gl.x, cfg.k, gl.store, gl.e2s, None, m.MOE_OUT_BF16)
    torch.cuda.synchronize()
    ref = o.moe_layer(gl.hi.x_bf16, gl.hi.logits[0], gl.weights.matrix, cfg.k, cfg.H, "a16", gl.e2s_np)
    np.testing.assert_array_equal(to_np(ids), ref["ids"])
    assert np.max(np.abs(to_np(w) - ref["w"])) <= W_TOL
    e32 = rel_err(to_np(out32), ref["out"])
    e16 = bf16_excess(to_np(out16), ref["out"])
    print(f"[{name}] invariant layer out fp32 rel {e32:.3e} bf16 excess {e16:.3e}", flush=True)
    assert e32 <= REL_TOL and e16 <= REL_TOL


def test_invariant_layer_token_alone_equals_batch_row():
    """Each of the 16 verify tokens through the one-call layer alone gives the
    output bits of its row when the 16 go through the same call together."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["verify16"]
    gl = GpuLayer(cfg)
    out_b, ids_b, w_b = m.moe_decode_layer_invariant(gl.logits, gl.x, cfg.k, gl.store, None, None, m.MOE_OUT_F32)
    torch.cuda.synchronize()
    for t in range(cfg.T):
        out, ids, w = m.moe_decode_layer_invariant(gl.logits[t:t + 1].contiguous(), gl.x[t:t + 1].contiguous(),
                                                   cfg.k, gl.store, None, None, m.MOE_OUT_F32)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_b[t:t + 1]) and torch.equal(w, w_b[t:t + 1]), t
        assert torch.equal(out.view(torch.int32), out_b[t:t + 1].view(torch.int32)), t


def test_invariant_layer_repeated_calls_and_graph():
    """Back-to-back calls and graph replays give the same bits (the workspace
    contents on entry do not matter)."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["decode1"]
    gl = GpuLayer(cfg)
    ws = torch.full((m.decode_layer_invariant_workspace_bytes(1, cfg.k, cfg.E, cfg.H, cfg.I),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    ref, _, _ = m.moe_decode_layer_invariant(gl.logits, gl.x, cfg.k, gl.store, None, None, m.MOE_OUT_F32, ws=ws)
    out = torch.empty_like(ref)
    ids = torch.empty((1, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, cfg.k), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.moe_decode_layer_invariant(gl.logits, gl.x, cfg.k, gl.store, None, None, m.MOE_OUT_F32, out, ids, w, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_decode_layer_invariant(gl.logits, gl.x, cfg.k, gl.store, None, None, m.MOE_OUT_F32, out, ids, w, ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
