"""GPU parity of the decode FFN over 3-bit per-row codebook experts
(moe_ffn_cb3_decode) against the fp64 oracle (ffn_cb3), through the C ABI.
Routing and bucketing come from moe_route / moe_permute (pinned elsewhere);
y_pair must be within 2e-3 of max|ref| (the decode arithmetic gives ~1e-7)."""
import numpy as np
import pytest
import torch

from gen import device as gd
from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": gi.CONFIGS["tiny"],
    "decode1": gi.CONFIGS["decode1"],
    "verify16": gi.CONFIGS["verify16"],
    # a routable subset smaller than E (expert_to_slot), several tokens per bucket
    "mid_resident": gi.custom("mid_resident", 768, 256, 40, 3, 9, seed=22, resident=12),
    # the largest hidden and expert width the kernels take
    "wide": gi.custom("wide", 6144, 4096, 8, 2, 3, seed=43),
    # expert width 2944: 92 index groups per down row, 64 in the full pass and
    # 28 left over, i.e. 4 x 28 = 112 (row, group) items in two passes
    "tail2": gi.custom("tail2", 512, 2944, 12, 3, 5, seed=44),
}


def _run(cfg, logits_np=None):
    import fp4_routed_expert_mxfp4_amd as m
    hi = gi.host_inputs(cfg)
    store = m.Cb3Store(*gd.fill_cb3_layer(cfg, 0, hi.resident[0]))
    x, logits, e2s = gd.upload(hi, 0)
    e2s_t = None if cfg.resident is None else e2s
    e2s_np = None if cfg.resident is None else hi.expert_to_slot[0]
    ids, w = m.moe_route(logits, cfg.k, e2s_t)
    off, sp, _ = m.moe_permute(ids, cfg.E)
    y = m.moe_ffn_cb3_decode(x, cfg.k, cfg.E, store, e2s_t, off, sp)
    torch.cuda.synchronize()
    ref_ids, _ = o.route(hi.logits[0], cfg.k, e2s_np)
    np.testing.assert_array_equal(to_np(ids), ref_ids)
    return hi, to_np(y), ref_ids, (store, x, off, sp, e2s_t)


@pytest.mark.parametrize("name", list(CASES))
def test_cb3_decode_matches_oracle(name):
    cfg = CASES[name]
    print(f"case {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    hi, y, ids, _ = _run(cfg)
    ref = o.ffn_cb3(hi.x_bf16, ids, gi.HostCb3Weights(cfg).matrix, cfg.H)
    e = rel_err(y, ref)
    print(f"[{name}] cb3 y_pair rel err {e:.3e}", flush=True)
    assert e <= REL_TOL
    assert e <= 1e-5  # fp32 sums of exact products: far inside the tolerance


def test_cb3_decode_deterministic():
    import fp4_routed_expert_mxfp4_amd as m
    cfg = CASES["verify16"]
    _, y1, _, (store, x, off, sp, e2s) = _run(cfg)
    y2 = to_np(m.moe_ffn_cb3_decode(x, cfg.k, cfg.E, store, e2s, off, sp))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_cb3_decode_graph_replays():
    """moe_ffn_cb3_decode captured in a HIP graph: three replays, with an eager
    call on other inputs between them, each bit-identical to the eager result."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = CASES["verify16"]
    _, y_eager, _, (store, x, off, sp, e2s) = _run(cfg)
    y = torch.empty((cfg.T * cfg.k, cfg.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(m.decode_workspace_bytes(cfg.T, cfg.k, cfg.I), 256), dtype=torch.uint8, device="cuda")
    other = torch.flip(x, dims=[0]).contiguous()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.moe_ffn_cb3_decode(x, cfg.k, cfg.E, store, e2s, off, sp, y, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_ffn_cb3_decode(x, cfg.k, cfg.E, store, e2s, off, sp, y, ws)
    for _ in range(3):
        m.moe_ffn_cb3_decode(other, cfg.k, cfg.E, store, e2s, off, sp, y, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(y).view(np.uint32), y_eager.view(np.uint32))
