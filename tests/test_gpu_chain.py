"""The 40-layer chained decode (154 of 384 experts resident per layer, bf16
residual stream, weightless RMS norm before each layer's MoE) against the
fp64 oracle.

* Every layer is one decode step: rmsnorm -> route over the layer's resident
  experts -> bucketing -> decode FFN -> combine with the residual.  Sampled
  layers are checked one by one on seeded inputs against the oracle's layer.
* The whole 40-layer chain runs as one captured HIP graph of
  moe_decode_layer_rmsnorm calls (the launch the benchmark times), bit-identical
  to the chain of separate calls.  Its first layers are compared with the oracle's own
  chain; over all 40 layers the routing must equal the oracle's exactly and
  the stream must stay finite and unit-normalised.
"""
import numpy as np
import pytest
import torch

from gen import device as gd
from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, bf16_excess, rel_err, to_np

pytestmark = pytest.mark.gpu

CFG = gi.CONFIGS["chain40"]


@pytest.fixture(scope="module")
def chain():
    import fp4_routed_expert_mxfp4_amd as m
    hi = gi.host_inputs(CFG)
    dev = torch.device("cuda")
    stores, logits, e2s = [], [], []
    for layer in range(CFG.layers):
        stores.append(m.ExpertStore(*gd.fill_layer(CFG, layer, hi.resident[layer])))
        logits.append(torch.from_numpy(hi.logits[layer]).to(dev))
        e2s.append(torch.from_numpy(hi.expert_to_slot[layer]).to(dev))
    yield hi, stores, logits, e2s
    del stores
    torch.cuda.empty_cache()


def layer_step(m, x, store, logits, e2s, ids, w, off, sp, p2r, y, ws, n, out, out32=None):
    k, E = CFG.k, CFG.E
    m.moe_rmsnorm_bf16(x, 1e-6, n)
    m.moe_route(logits, k, e2s, ids, w)
    m.moe_permute(ids, E, off, sp, p2r)
    m.moe_ffn_fp4_decode(n, k, E, store, e2s, off, sp, y, ws)
    m.moe_combine(y, w, x, m.MOE_OUT_BF16, out)
    if out32 is not None:
        m.moe_combine(y, w, x, m.MOE_OUT_F32, out32)


def buffers(m, layers=1):
    dev = torch.device("cuda")
    T, k, E, H = CFG.T, CFG.k, CFG.E, CFG.H
    return dict(
        ids=torch.empty((layers, T, k), dtype=torch.int32, device=dev),
        w=torch.empty((layers, T, k), dtype=torch.float32, device=dev),
        off=torch.empty((layers, E + 1), dtype=torch.int32, device=dev),
        sp=torch.empty((layers, T * k), dtype=torch.int32, device=dev),
        p2r=torch.empty((layers, T * k), dtype=torch.int32, device=dev),
        y=torch.empty((T * k, H), dtype=torch.float32, device=dev),
        ws=torch.empty(m.decode_workspace_bytes(T, k, CFG.I), dtype=torch.uint8, device=dev),
        n=torch.empty((T, H), dtype=torch.bfloat16, device=dev))


@pytest.mark.parametrize("layer", [0, 13, 26, 39])
def test_chain_layer_matches_oracle(chain, layer):
    """One chained layer on a seeded residual stream (magnitudes as the chain makes them)."""
    import fp4_routed_expert_mxfp4_amd as m
    hi, stores, logits, e2s = chain
    rng = np.random.default_rng(100 + layer)
    x_np = gi.f32_to_bf16_bits((rng.standard_normal((CFG.T, CFG.H)) * 3e5).astype(np.float32))
    x = torch.from_numpy(x_np.view(np.int16)).cuda().view(torch.bfloat16)
    b = buffers(m)
    out = torch.empty_like(x)
    out32 = torch.empty((CFG.T, CFG.H), dtype=torch.float32, device="cuda")
    layer_step(m, x, stores[layer], logits[layer], e2s[layer], b["ids"][0], b["w"][0], b["off"][0], b["sp"][0],
               b["p2r"][0], b["y"], b["ws"], b["n"], out, out32)
    torch.cuda.synchronize()
    hw = gi.HostWeights(CFG, layer)
    ref = o.chain_layer(x_np, hi.logits[layer], hw.matrix, CFG.k, CFG.H, hi.expert_to_slot[layer])
    np.testing.assert_array_equal(to_np(b["ids"][0]), ref["ids"])
    assert all(hi.expert_to_slot[layer][e] >= 0 for e in ref["ids"].reshape(-1))
    # the norm is a bf16 rounding of an fp32 (GPU) vs fp64 (oracle) value: at most one ulp apart
    nd = np.abs(to_np(b["n"]).astype(np.int32) - ref["norm"].astype(np.int32))
    assert nd.max() <= 1
    # the layer against the oracle's own chain step (its own norm, fp64 throughout)
    e32 = rel_err(to_np(out32), ref["out"])
    e16 = bf16_excess(to_np(out), ref["out"])
    print(f"[chain layer {layer}] out fp32 rel {e32:.3e} bf16 excess {e16:.3e}; norm ulp flips {np.count_nonzero(nd)}")
    assert e32 <= REL_TOL and e16 <= REL_TOL


def test_chain_40_layers_graph(chain):
    """The whole chain in one HIP graph, as the benchmark launches it (each layer one
    moe_decode_layer_rmsnorm call); eager, it equals the chain of separate calls bit for bit."""
    import fp4_routed_expert_mxfp4_amd as m
    hi, stores, logits, e2s = chain
    L = CFG.layers
    b = buffers(m, L)
    xs = [torch.from_numpy(hi.x_bf16.view(np.int16)).cuda().view(torch.bfloat16)]
    xs += [torch.empty((CFG.T, CFG.H), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    lws = torch.empty(m.decode_layer_rmsnorm_workspace_bytes(CFG.T, CFG.k, CFG.E, CFG.H, CFG.I), dtype=torch.uint8,
                      device="cuda")

    def token():
        for layer in range(L):
            m.moe_decode_layer_rmsnorm(logits[layer], xs[layer], CFG.k, stores[layer], 1e-6, e2s[layer],
                                       m.MOE_OUT_BF16, xs[layer + 1], b["ids"][layer], b["w"][layer], lws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        token()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [to_np(x) for x in xs]
    # the same chain as five separate calls per layer
    sep = [xs[0].clone()] + [torch.empty_like(xs[0]) for _ in range(L)]
    for layer in range(L):
        layer_step(m, sep[layer], stores[layer], logits[layer], e2s[layer], b["ids"][layer], b["w"][layer],
                   b["off"][layer], b["sp"][layer], b["p2r"][layer], b["y"], b["ws"], b["n"], sep[layer + 1])
    torch.cuda.synchronize()
    for layer in range(L + 1):
        assert np.array_equal(to_np(sep[layer]), eager[layer]), layer
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        token()
    for rep in range(3):
        for x in xs[1:]:
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        for layer in range(L + 1):
            assert np.array_equal(to_np(xs[layer]), eager[layer]), (rep, layer)
    ids = to_np(b["ids"])
    for layer in range(L):
        ref_ids, _ = o.route(hi.logits[layer], CFG.k, hi.expert_to_slot[layer])
        np.testing.assert_array_equal(ids[layer], ref_ids)
    fin = o.bf16_bits_to_f64(eager[L])
    assert np.all(np.isfinite(fin))
    # the oracle's own chain over the first three layers
    xr = hi.x_bf16
    for layer in range(3):
        ref = o.chain_layer(xr, hi.logits[layer], gi.HostWeights(CFG, layer).matrix, CFG.k, CFG.H,
                            hi.expert_to_slot[layer])
        e = bf16_excess(eager[layer + 1], ref["out"])
        print(f"[chain, layer {layer} of the oracle's own chain] bf16 excess {e:.3e}")
        assert e <= REL_TOL
        xr = ref["x_next"]
