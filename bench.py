#!/usr/bin/env python3
"""Throughput of the routed MoE FFN over MXFP4 experts on one MI355X.

Headline (value): single-layer decode at batch 1 -- hidden 5120, expert width
2304, 384 experts all resident, top-8 -- as achieved HBM GB/s of the whole
step (router, bucketing, decode FFN, combine), counting the algorithmic bytes
(the 8 routed experts' codes and scales, x, logits, output).  Each step uses
one of 64 logit sets in turn, so consecutive steps touch different experts
and the 256 MB last-level cache cannot hold the weights between them.  The
timed steps are one HIP graph of back-to-back layer calls, as a decode token
runs its layers; the same steps launched as one graph each are also reported.

Also reported: the gate/up kernel against the HBM roofline (HIP events on its
stream), the 4096-token prefill chunk (tokens/s of one layer) and the 40-layer
chained decode (154 of 384 experts resident per layer), and the fp64 CPU
oracle timed on a bounded sample on the host.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-FFN decode achieved HBM GB/s (% of peak); prefill tokens/s at 4096"
PEAK_HBM = 8.0e12          # bytes/s, MI355X published HBM3E bandwidth
PEAK_MXFP4 = 10.1e15       # FLOP/s, MI355X published dense MXFP4
MFMA_MEASURED = 8.4e15     # FLOP/s, the block-scaled e2m3 x e2m1 MFMA measured alone on one MI355X
NSETS = 64


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode1_gateup_traffic.md")
DECODE_SRC = os.path.join(ROOT, "fp4_routed_expert_mxfp4_amd", "csrc", "decode.hip")


def measured_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary,
    or None when that summary was taken on a different kernel source."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        src = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("source_sha256:", "traffic_bytes_per_launch:")))
    if fields.get("source_sha256", "").strip() != src:
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--chain-steps", type=int, default=30)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-chain", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-router-gate", action="store_true")
    ap.add_argument("--no-cb3", action="store_true")
    ap.add_argument("--only", choices=("decode", "prefill", "chain", "verify", "router", "cb3"), default=None,
                    help="run one section only (for profiling); prints that section's numbers")
    ap.add_argument("--calibrate", action="store_true",
                    help="only time torch's plain copy of 4 GiB (the HBM-bytes calibration kernel)")
    return ap.parse_args()


def layer_bytes(cfg, experts: int, T: int, out_bytes: int = 2) -> int:
    """Algorithmic bytes of one layer call: touched experts + x + logits + output."""
    return experts * cfg.expert_bytes + T * cfg.H * 2 + T * cfg.E * 4 + T * cfg.H * out_bytes


class DecodeBench:
    """Device state of the single-layer decode workload with 64 rotating routings."""

    def __init__(self, cfg, torch, m, gd, gi):
        self.cfg, self.torch, self.m = cfg, torch, m
        hi = gi.host_inputs(cfg)
        self.hi = hi
        self.store = m.ExpertStore(*gd.fill_layer(cfg, 0, hi.resident[0]))
        dev = torch.device("cuda")
        self.x, _, _ = gd.upload(hi, 0)
        sets = gi.logit_sets(cfg, hi.bias, NSETS)
        self.logit_sets = sets
        self.logits = torch.from_numpy(sets).to(dev)                  # [S][T][E]
        T, k, E = cfg.T, cfg.k, cfg.E
        i32, f32 = torch.int32, torch.float32
        self.ids = torch.empty((NSETS, T, k), dtype=i32, device=dev)
        self.w = torch.empty((NSETS, T, k), dtype=f32, device=dev)
        self.off = torch.empty((NSETS, E + 1), dtype=i32, device=dev)
        self.sp = torch.empty((NSETS, T * k), dtype=i32, device=dev)
        self.p2r = torch.empty((NSETS, T * k), dtype=i32, device=dev)
        self.y = torch.empty((T * k, cfg.H), dtype=f32, device=dev)
        self.ws = torch.empty(m.decode_workspace_bytes(T, k, cfg.I), dtype=torch.uint8, device=dev)
        self.lws = torch.empty(m.decode_layer_workspace_bytes(T, k, E, cfg.H, cfg.I), dtype=torch.uint8,
                               device=dev)
        self.out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
        # the two waves of the expert-subset runs: even expert ids, then odd ones
        even = (torch.arange(E, device=dev) % 2 == 0).to(torch.uint8)
        self.waves = (even, 1 - even)

    def step(self, s: int, phase: int = 0) -> None:
        """One decode layer in one call (two kernels at this shape)."""
        m, c = self.m, self.cfg
        m.moe_decode_layer(self.logits[s], self.x, c.k, self.store, None, None, m.MOE_OUT_BF16, self.out,
                           self.ids[s], self.w[s], self.lws, phase=phase)

    def gateup(self, s: int) -> None:
        self.step(s, 1)

    def down(self, s: int) -> None:
        self.step(s, 2)

    def step_separate(self, s: int) -> None:
        """The same layer as four separate calls (five kernels)."""
        m, c = self.m, self.cfg
        m.moe_route(self.logits[s], c.k, None, self.ids[s], self.w[s])
        m.moe_permute(self.ids[s], c.E, self.off[s], self.sp[s], self.p2r[s])
        m.moe_ffn_fp4_decode(self.x, c.k, c.E, self.store, None, self.off[s], self.sp[s], self.y, self.ws)
        m.moe_combine(self.y, self.w[s], None, m.MOE_OUT_BF16, self.out)

    def step_invariant(self, s: int) -> None:
        """The same layer as four calls with the batch-invariant decode FFN (a token's
        rows bit-identical alone or inside a verify batch)."""
        m, c = self.m, self.cfg
        m.moe_route(self.logits[s], c.k, None, self.ids[s], self.w[s])
        m.moe_permute(self.ids[s], c.E, self.off[s], self.sp[s], self.p2r[s])
        m.moe_ffn_fp4_decode_invariant(self.x, c.k, c.E, self.store, None, self.off[s], self.sp[s], self.y,
                                       self.ws)
        m.moe_combine(self.y, self.w[s], None, m.MOE_OUT_BF16, self.out)

    def step_two_wave(self, s: int) -> None:
        """The same layer with the expert FFN in two waves over complementary expert
        subsets (every expert's weights read once, y_pair bit-identical)."""
        m, c = self.m, self.cfg
        m.moe_route(self.logits[s], c.k, None, self.ids[s], self.w[s])
        m.moe_permute(self.ids[s], c.E, self.off[s], self.sp[s], self.p2r[s])
        for run in self.waves:
            m.moe_ffn_fp4_decode_subset(self.x, c.k, c.E, self.store, None, self.off[s], self.sp[s], run, self.y,
                                        self.ws)
        m.moe_combine(self.y, self.w[s], None, m.MOE_OUT_BF16, self.out)

    def touched(self) -> list[int]:
        """Distinct experts routed per set (host copy of the device routing)."""
        ids = self.ids.cpu().numpy()
        return [len(set(ids[s].reshape(-1).tolist())) for s in range(NSETS)]


def capture(torch, fn, count: int):
    """HIP graph holding fn(0..count-1) in order (one graph per call index)."""
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(count):
            fn(i)  # warm the launch path outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def capture_many(torch, fn, count: int):
    """One HIP graph holding fn(0), fn(1), ..., fn(count-1) back to back."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(count):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graphs(torch, graphs, steps: int, pick=lambda i, n: i % n) -> float:
    """Seconds for `steps` replays, HIP events on the replay stream."""
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        graphs[pick(i, len(graphs))].replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3


def decode_section(args, torch, m, gd, gi):
    cfg = gi.CONFIGS["decode1"]
    log(f"decode1: filling {cfg.E} experts ({cfg.E * cfg.expert_bytes / 1e9:.2f} GB)")
    db = DecodeBench(cfg, torch, m, gd, gi)
    for s in range(NSETS):
        db.step(s)
    torch.cuda.synchronize()
    touched = db.touched()
    # the timed steps are one HIP graph of back-to-back layer calls, as a decode
    # token runs its layers; step i uses routing i mod 64
    log("decode1: warmup")
    warm = capture_many(torch, lambda i: db.step(i % NSETS), max(args.warmup, 1))
    time_graphs(torch, [warm], 1)
    del warm
    log(f"decode1: timing {args.steps} steps")
    timed = capture_many(torch, lambda i: db.step(i % NSETS), args.steps)
    t = time_graphs(torch, [timed], 1)
    del timed
    per_step_bytes = [layer_bytes(cfg, touched[i % NSETS], cfg.T) for i in range(args.steps)]
    gbps = sum(per_step_bytes) / t / 1e9
    # for comparison: each step as its own graph launch (adds the launch gap)
    step_graphs = capture(torch, db.step, NSETS)
    time_graphs(torch, step_graphs, 16)
    per_launch_steps = min(args.steps, 512)
    t_launch = time_graphs(torch, step_graphs, per_launch_steps) / per_launch_steps
    del step_graphs
    # for comparison: the four separate calls, back to back in one graph
    sep_graph = capture_many(torch, lambda i: db.step_separate(i % NSETS), NSETS)
    time_graphs(torch, [sep_graph], 2)
    sep_reps = max(1, min(args.steps, 512) // NSETS)
    t_sep = time_graphs(torch, [sep_graph], sep_reps) / (sep_reps * NSETS)
    del sep_graph
    # the same four calls with the batch-invariant decode FFN
    inv_graph = capture_many(torch, lambda i: db.step_invariant(i % NSETS), NSETS)
    time_graphs(torch, [inv_graph], 2)
    t_inv = time_graphs(torch, [inv_graph], sep_reps) / (sep_reps * NSETS)
    del inv_graph
    # the gate/up kernel alone, then the down kernel alone: one graph of 64
    # back-to-back launches over the 64 routings, replayed; HIP events on the
    # replay stream bracket the whole timed region
    gu_graph = capture_many(torch, db.gateup, NSETS)
    dn_graph = capture_many(torch, db.down, NSETS)
    reps = max(1, max(args.steps, 256) // NSETS)
    time_graphs(torch, [gu_graph], 2)
    t_gu = time_graphs(torch, [gu_graph], reps) / (reps * NSETS)
    time_graphs(torch, [dn_graph], 2)
    t_dn = time_graphs(torch, [dn_graph], reps) / (reps * NSETS)
    # algorithmic bytes of each half: the k experts' weights, x or h, the logits, h, and the output
    gu_bytes = (cfg.k * (2 * cfg.I * (cfg.H // 2 + cfg.H // 32)) + cfg.H * 2 + cfg.E * 4
                + cfg.k * cfg.I * 4)
    dn_bytes = cfg.k * (cfg.H * (cfg.I // 2 + cfg.I // 32)) + cfg.k * cfg.I * 4 + cfg.H * 2
    res = dict(seconds=t, gbps=gbps, ms_per_step=t / args.steps * 1e3, touched_mean=sum(touched) / NSETS,
               gateup_us=t_gu * 1e6, gateup_bytes=gu_bytes, down_us=t_dn * 1e6, down_bytes=dn_bytes,
               separate_us=t_sep * 1e6, invariant_us=t_inv * 1e6, graph_per_step_us=t_launch * 1e6, db=db)
    log(f"decode1: {res['ms_per_step'] * 1e3:.1f} us/step, {gbps:.0f} GB/s (separate calls: {t_sep * 1e6:.1f} us; "
        f"separate calls, batch-invariant FFN: {t_inv * 1e6:.1f} us; "
        f"one graph launch per step: {t_launch * 1e6:.1f} us); "
        f"route+gate/up {t_gu * 1e6:.1f} us ({gu_bytes / t_gu / 1e9:.0f} GB/s), down+combine {t_dn * 1e6:.1f} us "
        f"({dn_bytes / t_dn / 1e9:.0f} GB/s)")
    return res


def cb3_section(args, torch, m, gd, gi, db=None):
    """The decode expert FFN over the 3-bit per-row codebook experts at decode1
    (moe_ffn_cb3_decode), beside moe_ffn_fp4_decode on the same 64 routings:
    each as one graph of 64 back-to-back FFN calls, replayed."""
    cfg = gi.CONFIGS["decode1"]
    if db is None:
        db = DecodeBench(cfg, torch, m, gd, gi)
    for s_ in range(NSETS):
        db.step_separate(s_)  # routing and buckets of every set
    log(f"cb3: filling {cfg.E} experts")
    cb = m.Cb3Store(*gd.fill_cb3_layer(cfg, 0, db.hi.resident[0]))
    k, E = cfg.k, cfg.E
    g_cb = capture_many(torch, lambda i: m.moe_ffn_cb3_decode(db.x, k, E, cb, None, db.off[i], db.sp[i], db.y,
                                                              db.ws), NSETS)
    g_fp = capture_many(torch, lambda i: m.moe_ffn_fp4_decode(db.x, k, E, db.store, None, db.off[i], db.sp[i],
                                                              db.y, db.ws), NSETS)
    reps = max(1, min(args.steps, 512) // NSETS)
    time_graphs(torch, [g_cb], 2)
    t_cb = time_graphs(torch, [g_cb], reps) / (reps * NSETS)
    time_graphs(torch, [g_fp], 2)
    t_fp = time_graphs(torch, [g_fp], reps) / (reps * NSETS)
    del g_cb, g_fp, cb
    ebytes = 2 * cfg.I * (cfg.H * 3 // 8 + 16) + cfg.H * (cfg.I * 3 // 8 + 16)
    nbytes = k * ebytes + cfg.H * 2 + k * cfg.H * 4
    fbytes = k * cfg.expert_bytes + cfg.H * 2 + k * cfg.H * 4
    log(f"cb3: FFN {t_cb * 1e6:.1f} us/token ({nbytes / t_cb / 1e9:.0f} GB/s of {nbytes / 1e6:.1f} MB); "
        f"FP4 FFN on the same routings {t_fp * 1e6:.1f} us ({fbytes / 1e6:.1f} MB)")
    return dict(ffn_us=t_cb * 1e6, bytes=nbytes, GBps=nbytes / t_cb / 1e9, frac_of_peak_hbm=nbytes / t_cb / PEAK_HBM,
                expert_bytes=ebytes, fp4_ffn_us_same_routings=t_fp * 1e6, fp4_bytes=fbytes)


def verify_section(args, torch, m, gd, gi):
    """The 16-token decode batch (Zipf-skewed routing: experts shared across
    tokens) through moe_decode_layer, over 64 rotating routings."""
    cfg = gi.CONFIGS["verify16"]
    log(f"verify16: filling {cfg.E} experts")
    db = DecodeBench(cfg, torch, m, gd, gi)
    for s in range(NSETS):
        db.step(s)
    torch.cuda.synchronize()
    touched = db.touched()
    steps = max(NSETS, min(args.steps, 512))
    g = capture_many(torch, lambda i: db.step(i % NSETS), steps)  # back to back, as in decode1
    time_graphs(torch, [g], 1)
    t = time_graphs(torch, [g], 1)
    del g
    nbytes = sum(layer_bytes(cfg, touched[i % NSETS], cfg.T) for i in range(steps))
    per = t / steps
    log(f"verify16: {per * 1e6:.1f} us/step, {nbytes / t / 1e9:.0f} GB/s, {sum(touched) / NSETS:.1f} experts/step")
    # the same steps as separate calls, and with the expert FFN in two waves (even, then odd expert ids)
    extra = {}
    for key, fn in (("separate_calls_us_per_step", db.step_separate), ("two_wave_us_per_step", db.step_two_wave)):
        g = capture_many(torch, lambda i: fn(i % NSETS), NSETS)
        time_graphs(torch, [g], 1)
        extra[key] = time_graphs(torch, [g], 2) / (2 * NSETS) * 1e6
        del g
    log(f"verify16: separate calls {extra['separate_calls_us_per_step']:.1f} us/step, expert FFN in two waves "
        f"{extra['two_wave_us_per_step']:.1f} us/step (same bytes)")
    return dict(us_per_step=per * 1e6, tokens_per_s=cfg.T / per, gbps=nbytes / t / 1e9,
                frac_of_peak_hbm=nbytes / t / PEAK_HBM, experts_touched_mean=sum(touched) / NSETS, **extra)


def read_ceiling(torch, gd) -> dict:
    """The measured streaming-read ceiling: the harness's probe kernel (every
    wavefront 16 KiB contiguous per step, all loads in flight) over 4 GiB
    resident in HBM, HIP events on its stream."""
    n = 4 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = gd.lib()
    stream = torch.cuda.current_stream()

    def run():
        assert L.gen_stream_read(a.data_ptr(), n, sink.data_ptr(), stream.cuda_stream) == 0

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del a
    torch.cuda.empty_cache()
    log(f"read ceiling: {n / t / 1e9:.0f} GB/s (streaming-read probe over 4 GiB)")
    return dict(bytes=n, us=t * 1e6, read_GBps=n / t / 1e9)


def prefill_section(args, torch, m, gd, gi):
    cfg = gi.CONFIGS["prefill4096"]
    hi = gi.host_inputs(cfg)
    log("prefill4096: filling experts")
    store = m.ExpertStore(*gd.fill_layer(cfg, 0, hi.resident[0]))
    x, logits, _ = gd.upload(hi, 0)
    dev = torch.device("cuda")
    T, k, E = cfg.T, cfg.k, cfg.E
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    p2r = torch.empty(T * k, dtype=torch.int32, device=dev)
    y = torch.empty((T * k, cfg.H), dtype=torch.float32, device=dev)
    ws = torch.empty(m.prefill_workspace_bytes(T, k, cfg.H, cfg.I), dtype=torch.uint8, device=dev)
    pws = torch.empty(max(m.permute_workspace_bytes(T, k, E), 256), dtype=torch.uint8, device=dev)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)

    def step(_i):
        m.moe_route(logits, k, None, ids, w)
        m.moe_permute(ids, E, off, sp, p2r, pws)
        m.moe_ffn_fp4_prefill(x, k, E, store, None, off, sp, y, ws)
        m.moe_combine(y, w, None, m.MOE_OUT_BF16, out)

    try:
        step(0)
        torch.cuda.synchronize()
    except m.MoeError as exc:
        log(f"prefill4096 skipped: {exc}")
        return None
    graphs = capture(torch, step, 1)
    time_graphs(torch, graphs, 3)
    t = time_graphs(torch, graphs, args.prefill_steps)
    per = t / args.prefill_steps
    flops = 6.0 * cfg.H * cfg.I * T * k
    touched = int((torch.diff(off) > 0).sum().item())
    wbytes = touched * cfg.expert_bytes
    binding = max(flops / PEAK_MXFP4, wbytes / PEAK_HBM)  # seconds at the binding roofline
    log(f"prefill4096: {per * 1e3:.3f} ms/layer, {T / per / 1e6:.2f} M tok/s, {touched} experts, "
        f"{wbytes / per / 1e9:.0f} GB/s of expert weights")
    return dict(ms_per_layer=per * 1e3, tokens_per_s=T / per, tflops=flops / per / 1e12,
                frac_of_mxfp4_peak=flops / per / PEAK_MXFP4,
                experts_touched=touched, weight_bytes=wbytes,
                weight_GBps=wbytes / per / 1e9, frac_of_peak_hbm_weights=wbytes / per / PEAK_HBM,
                frac_of_binding_roofline=binding / per, frac_of_measured_mfma=flops / per / MFMA_MEASURED)


def router_gate_section(args, torch, m, gd, gi):
    """moe_route_x (gate projection + top-k) at one token, the 16-token verify
    batch and the 4096-token chunk.  Each timed graph holds 40 back-to-back
    calls over 40 distinct W_r copies (one per layer of the chained decode),
    so no call finds its gate rows in cache from the previous one."""
    import numpy as np
    dev = torch.device("cuda")
    out = {}
    for name in ("decode1", "verify16", "prefill4096"):
        cfg = gi.CONFIGS[name]
        hi = gi.host_inputs(cfg)
        T, E, H, k = cfg.T, cfg.E, cfg.H, cfg.k
        x = torch.from_numpy(hi.x_bf16.view(np.int16)).to(dev)
        w0 = torch.from_numpy(gi.router_weights(cfg).view(np.int16)).to(dev)
        b_np = gi.router_bias(hi)
        b = None if b_np is None else torch.from_numpy(b_np).to(dev)
        layers = 40
        wl = [w0.clone() for _ in range(layers)]
        lg = torch.empty((T, E), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        tw = torch.empty((T, k), dtype=torch.float32, device=dev)
        g = capture_many(torch, lambda i: m.moe_route_x(x, wl[i], k, b, None, lg, ids, tw), layers)
        reps = 5 if T > 64 else 50
        time_graphs(torch, [g], 2)
        per = time_graphs(torch, [g], reps) / (reps * layers)
        nbytes = 2 * E * H + 2 * T * H + 4 * T * E + 8 * T * k
        flops = 2.0 * T * E * H
        out[name] = dict(us_per_call=per * 1e6, tokens=T, bytes=nbytes, GBps=nbytes / per / 1e9,
                         frac_of_peak_hbm=nbytes / per / PEAK_HBM, tflops=flops / per / 1e12,
                         kernels=("router_skinny_kernel" if T <= 64 else "router_mfma_kernel") + " + route_kernel")
        log(f"router gate {name}: {per * 1e6:.2f} us/call, {nbytes / per / 1e9:.0f} GB/s, "
            f"{flops / per / 1e12:.1f} TFLOP/s")
        del wl
    return out


def chain_section(args, torch, m, gd, gi):
    cfg = gi.CONFIGS["chain40"]
    hi = gi.host_inputs(cfg)
    dev = torch.device("cuda")
    log(f"chain40: filling {cfg.layers} x {cfg.resident} experts "
        f"({cfg.layers * cfg.resident * cfg.expert_bytes / 1e9:.1f} GB)")
    stores, logits, e2s = [], [], []
    for layer in range(cfg.layers):
        stores.append(m.ExpertStore(*gd.fill_layer(cfg, layer, hi.resident[layer])))
        logits.append(torch.from_numpy(hi.logits[layer]).to(dev))
        e2s.append(torch.from_numpy(hi.expert_to_slot[layer]).to(dev))
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    import numpy as np
    xs = [torch.from_numpy(hi.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)]
    xs += [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(cfg.layers)]
    ids = torch.empty((cfg.layers, T, k), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.layers, T, k), dtype=torch.float32, device=dev)
    off = torch.empty((cfg.layers, E + 1), dtype=torch.int32, device=dev)
    sp = torch.empty((cfg.layers, T * k), dtype=torch.int32, device=dev)
    ws = torch.empty(m.decode_layer_rmsnorm_workspace_bytes(T, k, E, H, cfg.I), dtype=torch.uint8, device=dev)

    def token(_i):  # each layer: RMS norm (inside the layer's first kernel) -> MoE -> + residual
        for layer in range(cfg.layers):
            m.moe_decode_layer_rmsnorm(logits[layer], xs[layer], k, stores[layer], 1e-6, e2s[layer], m.MOE_OUT_BF16,
                                       xs[layer + 1], ids[layer], w[layer], ws)

    graphs = capture(torch, token, 1)
    time_graphs(torch, graphs, 3)
    t = time_graphs(torch, graphs, args.chain_steps)
    per = t / args.chain_steps
    idn = ids.cpu().numpy()
    nbytes = sum(layer_bytes(cfg, len(set(idn[layer].reshape(-1).tolist())), T) + T * H * 2 * 2
                 for layer in range(cfg.layers))
    fin = xs[-1].float()
    finite = bool(torch.isfinite(fin).all().item())
    log(f"chain40: {per * 1e3:.3f} ms/token, {nbytes / per / 1e9:.0f} GB/s, finite={finite}")
    return dict(ms_per_token=per * 1e3, tokens_per_s=1.0 / per, gbps=nbytes / per / 1e9,
                frac_of_peak_hbm=nbytes / per / PEAK_HBM, bytes_per_token=nbytes, output_finite=finite)


def cpu_baseline(db, gi) -> dict:
    """The fp64 oracle on a bounded sample of the decode workload (3 routings)."""
    import numpy as np
    from oracle import moe_oracle as o
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = db.cfg
    hw = gi.HostWeights(cfg)
    n_tok, total_bytes, total_t = 10, 0, 0.0
    for s in range(n_tok):
        ids, _ = o.route(db.logit_sets[s], cfg.k)
        for e in set(ids.reshape(-1).tolist()):
            for mat in range(3):
                hw.matrix(int(e), mat)      # generate the inputs outside the timed region
        t0 = time.perf_counter()
        o.moe_layer(db.hi.x_bf16, db.logit_sets[s], hw.matrix, cfg.k, cfg.H)
        total_t += time.perf_counter() - t0
        total_bytes += layer_bytes(cfg, len(set(ids.reshape(-1).tolist())), cfg.T)
        hw.drop()
    log(f"cpu oracle: {total_t:.1f} s for {n_tok} decode tokens")
    return dict(value=total_bytes / total_t / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample=f"{n_tok} single-token decode layers of the same workload (logit sets 0-{n_tok - 1}), "
                       f"fp64 numpy oracle, weight generation excluded; {total_t:.1f} s",
                tokens_per_s=n_tok / total_t)


def calibrate(torch) -> dict:
    """Plain device copy of 4 GiB (torch's copy kernel): a measured streaming
    ceiling and the known-size kernel the HBM byte counters are scaled by."""
    n = 4 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    res = dict(bytes_read=n, bytes_written=n, us=t * 1e6, copy_GBps=2 * n / t / 1e9)
    log(f"calibration copy: {t * 1e6:.0f} us per 4 GiB copy, {2 * n / t / 1e9:.0f} GB/s read+write")
    return res


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        print("bench.py: only --gpus 1 is supported (the path is built and measured on one GPU)",
              file=sys.stderr)
        return 2
    import torch
    import fp4_routed_expert_mxfp4_amd as m
    from gen import device as gd
    from gen import inputs as gi
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    m.lib()
    if args.calibrate:
        print(json.dumps({"calibration": calibrate(torch)}), flush=True)
        return 0

    if args.only:
        fn = {"decode": decode_section, "prefill": prefill_section, "chain": chain_section,
              "verify": verify_section, "router": router_gate_section, "cb3": cb3_section}[args.only]
        res = fn(args, torch, m, gd, gi)
        if isinstance(res, dict):
            res.pop("db", None)
        print(json.dumps({"section": args.only, "result": res}), flush=True)
        return 0

    ceiling = read_ceiling(torch, gd)
    dec = decode_section(args, torch, m, gd, gi)
    cfg = gi.CONFIGS["decode1"]
    verify = None if args.no_verify else verify_section(args, torch, m, gd, gi)
    prefill = None if args.no_prefill else prefill_section(args, torch, m, gd, gi)
    chain = None if args.no_chain else chain_section(args, torch, m, gd, gi)
    router = None if args.no_router_gate else router_gate_section(args, torch, m, gd, gi)
    cb3 = None if args.no_cb3 else cb3_section(args, torch, m, gd, gi, dec["db"])
    cpu = None if args.no_cpu_baseline else cpu_baseline(dec["db"], gi)

    gu_achieved = dec["gateup_bytes"] / (dec["gateup_us"] * 1e-6)
    result = {
        "metric": METRIC,
        "value": round(dec["gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "decode1: single-layer MoE FFN decode, batch 1, hidden 5120, expert width 2304, "
                               "384 MXFP4 experts resident, top-8, 64 rotating routings",
                   "hidden": cfg.H, "expert_width": cfg.I, "experts": cfg.E, "top_k": cfg.k, "tokens": cfg.T,
                   "weights": "e2m1 + UE8M0/32", "activations": "bf16"},
        "frac_of_peak_hbm": round(dec["gbps"] * 1e9 / PEAK_HBM, 4),
        "separate_calls_us_per_step": round(dec["separate_us"], 2),
        "batch_invariant_separate_calls_us_per_step": round(dec["invariant_us"], 2),
        "graph_launch_per_step_us": round(dec["graph_per_step_us"], 2),
        "roofline": {"kernel": "decode route + gate/up + SwiGLU (fused_gateup_kernel, moe_decode_layer_gateup)",
                     "bound": "hbm",
                     "achieved": round(gu_achieved / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(gu_achieved / PEAK_HBM, 4), "traffic": measured_traffic(),
                     "avg_us": round(dec["gateup_us"], 2), "bytes_per_launch": dec["gateup_bytes"]},
        "down_kernel": {"kernel": "decode down + combine (fused_down_combine_kernel, moe_decode_layer_down)",
                        "avg_us": round(dec["down_us"], 2), "bytes_per_launch": dec["down_bytes"],
                        "achieved_GBps": round(dec["down_bytes"] / dec["down_us"] / 1e3, 1)},
        "cpu_baseline": cpu,
        "measured_read_ceiling_GBps": round(ceiling["read_GBps"], 1),
        "verify16": verify,
        "prefill4096": prefill,
        "chain40": chain,
        "router_gate": router,
        "cb3_decode1": cb3,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
