"""GPU parity of the router gate projection (moe_router_logits, moe_route_x)
against the fp64 oracle, through the C ABI.

Logits: every element within the rigorous bound of fp32 summation of exact
bf16 products, (H + 1) * 2^-24 * (sum_c |x_c w_c| + |b|) / (1 - (H + 1) 2^-24),
whatever the order of the sums, and max|err| / max|ref| <= 1e-5 overall.
Routing: the selection is an integer decided by floating point, so the ids
must equal the oracle's bit for bit on every token whose ranking among its
first k + 1 candidates is separated by more than the logits' error bound;
on a token with a closer call (none is expected at these sizes) the GPU's
pick must be a valid top-k within that bound.  The GPU's ids and weights
must also be exactly what moe_route writes for the GPU's own logits.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import to_np

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24

CASES = {
    # name: (config, routable-subset size or None)
    "tiny": (gi.CONFIGS["tiny"], None),                                       # GEMV, half-filled 512-step
    "decode1": (gi.CONFIGS["decode1"], None),                                 # GEMV, one token
    "verify16": (gi.CONFIGS["verify16"], None),                               # GEMV, Zipf bias
    "gemv64": (gi.custom("gemv64", 1024, 128, 48, 6, 64, seed=31, zipf=1.1), 30),  # largest GEMV batch, masked
    "mfma65": (gi.custom("mfma65", 512, 128, 384, 8, 65, seed=32, zipf=1.1), None),  # MFMA, ragged token tile
    "mfma_e8": (gi.custom("mfma_e8", 256, 128, 8, 2, 100, seed=33), 5),       # one partial expert fragment
    "mfma_e40": (gi.custom("mfma_e40", 768, 128, 40, 4, 200, seed=34, zipf=1.1), None),  # E % 16 != 0
    "mfma_e500": (gi.custom("mfma_e500", 512, 128, 500, 8, 130, seed=35), None),   # four expert tiles
    "mfma_e1024": (gi.custom("mfma_e1024", 256, 128, 1024, 16, 96, seed=36), 700),  # largest E, eight expert tiles
}


def _inputs(cfg, n_res, device="cuda"):
    hi = gi.host_inputs(cfg)
    w_np = gi.router_weights(cfg)
    b_np = gi.router_bias(hi)
    e2s_np = None
    if n_res is not None:
        rng = np.random.default_rng(cfg.seed + 77)
        keep = np.sort(rng.choice(cfg.E, n_res, replace=False))
        e2s_np = np.full(cfg.E, -1, np.int32)
        e2s_np[keep] = np.arange(n_res, dtype=np.int32)
    dev = torch.device(device)
    x = torch.from_numpy(hi.x_bf16.view(np.int16)).to(dev)
    w = torch.from_numpy(w_np.view(np.int16)).to(dev)
    b = None if b_np is None else torch.from_numpy(b_np).to(dev)
    e2s = None if e2s_np is None else torch.from_numpy(e2s_np).to(dev)
    return hi, w_np, b_np, e2s_np, x, w, b, e2s


def _bound(hi, w_np, b_np):
    """Per-element error bound of an fp32 sum of exact products, any order."""
    H = hi.cfg.H
    xa = np.abs(o.bf16_bits_to_f64(hi.x_bf16))
    wa = np.abs(o.bf16_bits_to_f64(w_np))
    mag = xa @ wa.T
    if b_np is not None:
        mag = mag + np.abs(b_np.astype(np.float64))[None, :]
    n = H + 1
    return n * U32 * mag / (1 - n * U32)


def _check_routing(name, ref_l, bound, ids, w, k, e2s_np):
    T, E = ref_l.shape
    ref_ids, ref_w = o.route(ref_l.astype(np.float32), k, e2s_np)
    routable = np.ones(E, bool) if e2s_np is None else e2s_np >= 0
    close = 0
    for t in range(T):
        cand = np.nonzero(routable)[0]
        order = cand[np.lexsort((cand, -ref_l[t, cand]))][:k + 1]
        gaps = -np.diff(ref_l[t, order])
        need = bound[t, order[:-1]] + bound[t, order[1:]] + 2 * U32 * np.abs(ref_l[t, order[:-1]])
        if np.all(gaps > need):
            np.testing.assert_array_equal(ids[t], ref_ids[t], err_msg=f"{name} token {t}")
            assert np.max(np.abs(w[t] - ref_w[t])) <= 1e-6 + np.max(bound[t])
        else:
            close += 1
            assert len(set(ids[t].tolist())) == k and np.all(routable[ids[t]])
            kth = ref_l[t, order[k - 1]]
            assert np.all(ref_l[t, ids[t]] >= kth - 2 * np.max(bound[t]))
    assert np.max(np.abs(w.sum(1) - 1.0)) <= 1e-6
    return close


@pytest.mark.parametrize("name", list(CASES))
def test_router_gate_matches_oracle(name):
    import fp4_routed_expert_mxfp4_amd as m
    cfg, n_res = CASES[name]
    print(f"case {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}", flush=True)
    hi, w_np, b_np, e2s_np, x, w, b, e2s = _inputs(cfg, n_res)
    lg = m.moe_router_logits(x, w, b)
    l2, ids, tw = m.moe_route_x(x, w, cfg.k, b, e2s)
    ids_r, tw_r = m.moe_route(l2, cfg.k, e2s)
    torch.cuda.synchronize()
    lg, l2 = to_np(lg), to_np(l2)
    ids, tw, ids_r, tw_r = to_np(ids), to_np(tw), to_np(ids_r), to_np(tw_r)
    # the two calls compute the same logits; route_x's top-k is moe_route's on them
    np.testing.assert_array_equal(lg.view(np.uint32), l2.view(np.uint32))
    np.testing.assert_array_equal(ids, ids_r)
    np.testing.assert_array_equal(tw.view(np.uint32), tw_r.view(np.uint32))
    ref = o.router_logits(hi.x_bf16, w_np, b_np)
    bound = _bound(hi, w_np, b_np)
    err = np.abs(l2.astype(np.float64) - ref)
    rel = float(np.max(err) / np.max(np.abs(ref)))
    close = _check_routing(name, ref, bound, ids, tw, cfg.k, e2s_np)
    print(f"[{name}] logits max err {np.max(err):.3e} rel {rel:.3e} (bound used {np.max(err / bound):.3f}); "
          f"close calls {close}", flush=True)
    assert np.all(err <= bound)
    assert rel <= 1e-5


def test_router_gate_prefill4096_full():
    """The 4096-token chunk at the model's shape: every logit and every token's routing."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.CONFIGS["prefill4096"]
    print("case prefill4096 router gate", flush=True)
    hi, w_np, b_np, _, x, w, b, _ = _inputs(cfg, None)
    l, ids, tw = m.moe_route_x(x, w, cfg.k, b)
    torch.cuda.synchronize()
    l, ids, tw = to_np(l), to_np(ids), to_np(tw)
    ref = o.router_logits(hi.x_bf16, w_np, b_np)
    bound = _bound(hi, w_np, b_np)
    err = np.abs(l.astype(np.float64) - ref)
    assert np.all(err <= bound)
    assert float(np.max(err) / np.max(np.abs(ref))) <= 1e-5
    close = _check_routing("prefill4096", ref, bound, ids, tw, cfg.k, None)
    print(f"[prefill4096] logits max err {np.max(err):.3e}; close calls {close}", flush=True)


def test_router_gate_deterministic_and_empty():
    """Two calls give the same bytes; T = 0 enqueues nothing and succeeds."""
    import fp4_routed_expert_mxfp4_amd as m
    for name in ("decode1", "mfma65"):
        cfg, n_res = CASES[name]
        _, _, _, _, x, w, b, e2s = _inputs(cfg, n_res)
        a = m.moe_route_x(x, w, cfg.k, b, e2s)
        c = m.moe_route_x(x, w, cfg.k, b, e2s)
        torch.cuda.synchronize()
        for u, v in zip(a, c):
            assert torch.equal(u.view(torch.int32), v.view(torch.int32))
    x0 = torch.empty((0, 256), dtype=torch.int16, device="cuda")
    w0 = torch.zeros((8, 256), dtype=torch.int16, device="cuda")
    l0, i0, t0 = m.moe_route_x(x0, w0, 2)
    assert l0.shape == (0, 8) and i0.shape == (0, 2)


def test_route_x_graph_replays():
    """moe_route_x captured in a HIP graph: three replays, with eager calls on
    other inputs between them, each bit-identical to the eager result."""
    import fp4_routed_expert_mxfp4_amd as m
    for name in ("verify16", "mfma65"):
        cfg, n_res = CASES[name]
        print(f"case {name} graph", flush=True)
        _, _, _, _, x, w, b, e2s = _inputs(cfg, n_res)
        lg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
        ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
        tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
        ref = [t.clone() for t in m.moe_route_x(x, w, cfg.k, b, e2s, lg, ids, tw)]
        other = torch.flip(x, dims=[0]).contiguous()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            m.moe_route_x(x, w, cfg.k, b, e2s, lg, ids, tw)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            m.moe_route_x(x, w, cfg.k, b, e2s, lg, ids, tw)
        for _ in range(3):
            m.moe_route_x(other, w, cfg.k, b, e2s, lg, ids, tw)   # eager work that overwrites the outputs
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for got, want in zip((lg, ids, tw), ref):
                assert torch.equal(got.view(torch.int32), want.view(torch.int32))
