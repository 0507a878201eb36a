"""The four-call layer (moe_route -> moe_permute -> expert FFN -> moe_combine)
captured in one HIP graph, for the prefill path and the multi-token decode
path: three replays, each after eager calls on other inputs that overwrite
every buffer, must reproduce the eager result bit for bit (routing, bucket
order, y_pair and the combined output)."""
import pytest
import torch

from gen import inputs as gi
from tests.harness import GpuLayer

pytestmark = pytest.mark.gpu

CASES = {
    # prefill: tiled and small-bucket paths, ragged tiles
    "prefill_mid_zipf": ("prefill", gi.custom("graph_prefill", 1024, 384, 24, 4, 300, seed=51, zipf=1.1)),
    # multi-token decode (MFMA path), masked routable subset
    "decode_mt16": ("decode", gi.custom("graph_decode", 1024, 256, 32, 4, 16, seed=52, zipf=1.1, resident=20)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_graph_replays(name):
    import fp4_routed_expert_mxfp4_amd as m
    path, cfg = CASES[name]
    print(f"case {name}: {path} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    gl = GpuLayer(cfg)
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    dev = gl.x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    p2r = torch.empty(T * k, dtype=torch.int32, device=dev)
    pws = torch.empty(max(m.moe.permute_workspace_bytes(T, k, E), 256), dtype=torch.uint8, device=dev)
    y = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    need = (m.prefill_workspace_bytes(T, k, H, cfg.I) if path == "prefill"
            else m.decode_workspace_bytes(T, k, cfg.I))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ffn = m.moe_ffn_fp4_prefill if path == "prefill" else m.moe_ffn_fp4_decode
    xa, la = gl.x, gl.logits
    xb, lb = torch.flip(xa, dims=[0]).contiguous(), torch.flip(la, dims=[0]).contiguous()
    src_x, src_l = xa.clone(), la.clone()  # the graph reads these buffers

    def layer():
        m.moe_route(src_l, k, gl.e2s, ids, w)
        m.moe_permute(ids, E, off, sp, p2r, pws)
        ffn(src_x, k, E, gl.store, gl.e2s, off, sp, y, ws)
        m.moe_combine(y, w, None, m.MOE_OUT_F32, out)

    layer()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (ids, w, off, sp, y, out)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(3):
        src_x.copy_(xb)
        src_l.copy_(lb)
        layer()  # eager work on other inputs through the same buffers
        torch.cuda.synchronize()
        src_x.copy_(xa)
        src_l.copy_(la)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((ids, w, off, sp, y, out), ref, ("ids", "w", "offsets", "sorted_pair", "y", "out")):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"replay {rep}: {what}"
    print(f"[{name}] three replays bit-identical to eager", flush=True)
