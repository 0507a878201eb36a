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


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_utilisation.md")
PREFILL_SRC = os.path.join(ROOT, "fp4_routed_expert_mxfp4_amd", "csrc", "prefill.hip")


def profile_fields(path: str, src: str, keys) -> dict | None:
    """`key: value` lines of a committed profile summary, or None when the
    summary was taken on a different kernel source."""
    import hashlib
    try:
        text = open(path).read()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith(" "))
    if fields.get("source_sha256", "").strip() != sha:
        return None
    out = {}
    for k in keys:
        try:
            out[k] = float(fields[k])
        except (KeyError, ValueError):
            out[k] = None
    return out


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-steps", type=int, default=60)
    ap.add_argument("--chain-steps", type=int, default=30)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-chain", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-router-gate", action="store_true")
    ap.add_argument("--no-cb3", action="store_true")
    ap.add_argument("--no-series", action="store_true",
                    help="skip the per-replay, cache-flushed and interleaved series (for counter runs)")
    ap.add_argument("--only", choices=("decode", "prefill", "chain", "verify", "router", "cb3"), default=None,
                    help="run one section only (for profiling); prints that section's numbers")
    ap.add_argument("--load-probe", action="store_true",
                    help="only measure the per-CU rate of the weight-tile load shapes (gen_load_probe)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run the two HBM-bytes calibration kernels (a 4 GiB copy and a 4 GiB read)")
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
        self.iws = torch.empty(m.decode_layer_invariant_workspace_bytes(T, k, E, cfg.H, cfg.I), dtype=torch.uint8,
                               device=dev)
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

    def step_invariant_layer(self, s: int) -> None:
        """The same layer on the batch-invariant arithmetic in one call
        (moe_decode_layer_invariant)."""
        m, c = self.m, self.cfg
        m.moe_decode_layer_invariant(self.logits[s], self.x, c.k, self.store, None, None, m.MOE_OUT_BF16, self.out,
                                     self.ids[s], self.w[s], self.iws)

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


FLUSH_BYTES = 512 << 20    # read before each cold replay: twice the 256 MB last-level cache
REPLAYS = 60               # replays of each per-replay series (median and min reported)


def provenance() -> dict:
    """Source hash, git commit (when a checkout is present), seeds and versions.
    Taken before the GPU is touched (the git query runs as a child process)."""
    import hashlib
    import platform
    import subprocess
    h = hashlib.sha256()
    for d in (os.path.join("fp4_routed_expert_mxfp4_amd", "csrc"), "include", "gen"):
        for f in sorted(os.listdir(os.path.join(ROOT, d))):
            if f.endswith((".hip", ".cuh", ".cpp", ".h", ".py")):
                h.update(f"{d}/{f}".encode())
                with open(os.path.join(ROOT, d, f), "rb") as fh:
                    h.update(fh.read())
    sha = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=20)
        sha = r.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    from gen import inputs as gi
    built = None
    try:
        with open(os.path.join(ROOT, "fp4_routed_expert_mxfp4_amd", "build_info.json")) as f:
            built = json.load(f)
    except (OSError, ValueError):
        pass
    return dict(git_sha=sha, source_sha256=h.hexdigest(), libraries_built_from=built, host=platform.node(), python=platform.python_version(),
                seeds={name: c.seed for name, c in gi.CONFIGS.items()},
                inputs="gen/inputs.py (PCG64 host draws) + gen/splitmix.py (SplitMix64 weight codes and scales)")


def stats_us(per_step_s: list) -> dict:
    import statistics
    v = sorted(x * 1e6 for x in per_step_s)
    return dict(n=len(v), median_us=round(statistics.median(v), 3), min_us=round(v[0], 3), max_us=round(v[-1], 3),
                mean_us=round(sum(v) / len(v), 3))


class Clock:
    """The shader clock while busy: a probe kernel of 256 one-wavefront
    workgroups compares the shader cycle counter with the constant 100 MHz
    counter over ~70 us of dependent arithmetic (no child process: the
    program has the GPU open)."""

    def __init__(self, torch, gd):
        self.torch, self.L = torch, gd.lib()
        self.out = torch.zeros(512, dtype=torch.int64, device="cuda")

    def read(self) -> dict:
        torch = self.torch
        stream = torch.cuda.current_stream()
        assert self.L.gen_clock_probe(self.out.data_ptr(), 256, 4000, stream.cuda_stream) == 0
        torch.cuda.synchronize()
        v = self.out.view(256, 2).cpu().tolist()
        mhz = sorted(100.0 * c / r for c, r in v if r > 0)
        return dict(probe_sclk_mhz_median=round(mhz[len(mhz) // 2], 1), probe_sclk_mhz_min=round(mhz[0], 1))


def replay_series(torch, graph, steps_per_replay: int, reps: int, flush=None) -> list:
    """Seconds per step of each of `reps` replays of `graph`, each bracketed by
    HIP events on the replay stream; flush() runs before each replay, outside
    the bracket."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / 1e3 / steps_per_replay for a, b in ev]


def interleaved(torch, arms: dict, steps_per_replay: int, rounds: int) -> dict:
    """Replays the arms' graphs in turn (A B C A B C ...), each replay bracketed
    by HIP events; per-step median and min of each arm."""
    per = {k: [] for k in arms}
    for _ in range(rounds):
        for k, g in arms.items():
            per[k] += replay_series(torch, g, steps_per_replay, 1)
    return {k: stats_us(v) for k, v in per.items()}


def make_flush(torch, gd):
    buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = gd.lib()

    def flush():
        assert L.gen_stream_read(buf.data_ptr(), FLUSH_BYTES, sink.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream) == 0
    return flush


def decode_section(args, torch, m, gd, gi):
    cfg = gi.CONFIGS["decode1"]
    log(f"decode1: filling {cfg.E} experts ({cfg.E * cfg.expert_bytes / 1e9:.2f} GB)")
    db = DecodeBench(cfg, torch, m, gd, gi)
    for s in range(NSETS):
        db.step(s)
    torch.cuda.synchronize()
    touched = db.touched()
    clk = Clock(torch, gd)
    clock_before = clk.read()
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
    mean_bytes = sum(layer_bytes(cfg, touched[i], cfg.T) for i in range(NSETS)) / NSETS
    series = not args.no_series
    # per-replay series: a graph of the 64 routings back to back, each replay
    # bracketed by its own events (median and min over the replays)
    rep = capture_many(torch, lambda i: db.step(i % NSETS), NSETS)
    replay_series(torch, rep, NSETS, 2)
    replays = stats_us(replay_series(torch, rep, NSETS, REPLAYS if series else 3))
    # cold series: one step per replay, after a 512 MiB read that evicts the
    # last-level cache (routing i mod 64, one graph per routing)
    step_graphs = capture(torch, db.step, NSETS)
    flush = make_flush(torch, gd)
    cold_s = []
    for r in range(REPLAYS if series else 3):
        cold_s += replay_series(torch, step_graphs[r % NSETS], 1, 1, flush)
    cold = stats_us(cold_s)
    # for comparison: each step as its own graph launch (adds the launch gap)
    time_graphs(torch, step_graphs, 16)
    per_launch_steps = min(args.steps, 512)
    t_launch = time_graphs(torch, step_graphs, per_launch_steps) / per_launch_steps
    del step_graphs
    # the four separate calls and the four calls with the batch-invariant FFN,
    # interleaved with the one-call layer (A B C A B C ...)
    sep_graph = capture_many(torch, lambda i: db.step_separate(i % NSETS), NSETS)
    inv_graph = capture_many(torch, lambda i: db.step_invariant(i % NSETS), NSETS)
    invl_graph = capture_many(torch, lambda i: db.step_invariant_layer(i % NSETS), NSETS)
    for g in (sep_graph, inv_graph, invl_graph):
        time_graphs(torch, [g], 2)
    ab = interleaved(torch, {"layer": rep, "separate_calls": sep_graph, "invariant_separate_calls": inv_graph,
                             "invariant_layer": invl_graph}, NSETS, 20 if series else 1)
    t_sep = ab["separate_calls"]["median_us"] * 1e-6
    t_inv = ab["invariant_separate_calls"]["median_us"] * 1e-6
    t_invl = ab["invariant_layer"]["median_us"] * 1e-6
    del sep_graph, inv_graph, invl_graph, rep
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
    gu_rep = stats_us(replay_series(torch, gu_graph, NSETS, REPLAYS if series else 3))
    del gu_graph, dn_graph
    clock_after = clk.read()
    # algorithmic bytes of each half: the k experts' weights, x or h, the logits, h, and the output
    gu_bytes = (cfg.k * (2 * cfg.I * (cfg.H // 2 + cfg.H // 32)) + cfg.H * 2 + cfg.E * 4
                + cfg.k * cfg.I * 4)
    dn_bytes = cfg.k * (cfg.H * (cfg.I // 2 + cfg.I // 32)) + cfg.k * cfg.I * 4 + cfg.H * 2
    res = dict(seconds=t, gbps=gbps, ms_per_step=t / args.steps * 1e3, touched_mean=sum(touched) / NSETS,
               gateup_us=t_gu * 1e6, gateup_bytes=gu_bytes, down_us=t_dn * 1e6, down_bytes=dn_bytes,
               separate_us=t_sep * 1e6, invariant_us=t_inv * 1e6, invariant_layer_us=t_invl * 1e6,
               graph_per_step_us=t_launch * 1e6,
               replays=dict(replays, GBps_at_median=round(mean_bytes / (replays["median_us"] * 1e-6) / 1e9, 1)),
               cold=dict(cold, GBps_at_median=round(mean_bytes / (cold["median_us"] * 1e-6) / 1e9, 1),
                         flush_bytes=FLUSH_BYTES),
               interleaved=ab, gateup_replays=gu_rep, clocks=dict(before=clock_before, after=clock_after), db=db)
    log(f"decode1: {res['ms_per_step'] * 1e3:.1f} us/step, {gbps:.0f} GB/s; per replay of 64 steps median "
        f"{replays['median_us']:.1f} min {replays['min_us']:.1f} us/step; cold (LLC flushed) median "
        f"{cold['median_us']:.1f} us; interleaved medians: layer {ab['layer']['median_us']:.1f}, separate calls "
        f"{t_sep * 1e6:.1f}, batch-invariant separate calls {t_inv * 1e6:.1f}, batch-invariant layer "
        f"{t_invl * 1e6:.1f} us; one graph launch per step "
        f"{t_launch * 1e6:.1f} us; route+gate/up {t_gu * 1e6:.1f} us ({gu_bytes / t_gu / 1e9:.0f} GB/s), "
        f"down+combine {t_dn * 1e6:.1f} us ({dn_bytes / t_dn / 1e9:.0f} GB/s); sclk "
        f"{clock_before['probe_sclk_mhz_median']:.0f} -> {clock_after['probe_sclk_mhz_median']:.0f} MHz")
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
    clk = Clock(torch, gd)
    clock_before = clk.read()
    g = capture_many(torch, lambda i: db.step(i % NSETS), steps)  # back to back, as in decode1
    time_graphs(torch, [g], 1)
    t = time_graphs(torch, [g], 1)
    del g
    g = capture_many(torch, lambda i: db.step(i % NSETS), NSETS)
    replay_series(torch, g, NSETS, 2)
    replays = stats_us(replay_series(torch, g, NSETS, REPLAYS if not args.no_series else 3))
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
    clock_after = clk.read()
    log(f"verify16: separate calls {extra['separate_calls_us_per_step']:.1f} us/step, expert FFN in two waves "
        f"{extra['two_wave_us_per_step']:.1f} us/step (same bytes); per replay of 64 steps median "
        f"{replays['median_us']:.1f} min {replays['min_us']:.1f} us/step")
    return dict(us_per_step=per * 1e6, tokens_per_s=cfg.T / per, gbps=nbytes / t / 1e9,
                frac_of_peak_hbm=nbytes / t / PEAK_HBM, experts_touched_mean=sum(touched) / NSETS, **extra,
                replays=replays, clocks=dict(before=clock_before, after=clock_after))


def read_ceiling(torch, gd, lds: bool = False) -> dict:
    """The measured streaming-read ceiling: the harness's probe kernel (every
    wavefront 16 KiB contiguous per step, all loads in flight; with lds the
    loads are copies into LDS by the buffer unit) over 4 GiB resident in HBM,
    HIP events on its stream."""
    n = 4 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = gd.lib()
    stream = torch.cuda.current_stream()

    def run():
        fn = L.gen_stream_read_lds if lds else L.gen_stream_read
        assert fn(a.data_ptr(), n, sink.data_ptr(), stream.cuda_stream) == 0

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
    log(f"read ceiling: {n / t / 1e9:.0f} GB/s (streaming-read probe over 4 GiB{', copies into LDS' if lds else ''})")
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
    # the experts' copy in MFMA operand order for the tiled GEMMs, made once when the
    # experts are loaded (outside the timed step, like the experts themselves)
    packed = torch.empty(m.prefill_packed_bytes(store.num_slots, cfg.H, cfg.I), dtype=torch.uint8, device=dev)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    m.moe_prefill_pack_weights(store, packed)
    p1.record()
    torch.cuda.synchronize()
    pack_ms = p0.elapsed_time(p1)

    def step_with(ffn):
        def step(_i):
            m.moe_route(logits, k, None, ids, w)
            m.moe_permute(ids, E, off, sp, p2r, pws)
            ffn()
            m.moe_combine(y, w, None, m.MOE_OUT_BF16, out)
        return step

    step = step_with(lambda: m.moe_ffn_fp4_prefill_packed(x, k, E, store, packed, None, off, sp, y, ws))
    step_rm = step_with(lambda: m.moe_ffn_fp4_prefill(x, k, E, store, None, off, sp, y, ws))
    try:
        step(0)
        torch.cuda.synchronize()
    except m.MoeError as exc:
        log(f"prefill4096 skipped: {exc}")
        return None
    clk = Clock(torch, gd)
    clock_before = clk.read()
    graphs = capture(torch, step, 1)
    time_graphs(torch, graphs, 3)
    t = time_graphs(torch, graphs, args.prefill_steps)
    per = t / args.prefill_steps
    series = not args.no_series
    replays = stats_us(replay_series(torch, graphs[0], 1, max(REPLAYS, args.prefill_steps) if series else 3))
    flush = make_flush(torch, gd)
    cold = stats_us(replay_series(torch, graphs[0], 1, 20 if series else 3, flush))
    clock_after = clk.read()
    del graphs
    # the same step with the tiled GEMMs on the row-major store (no packed copy)
    graphs_rm = capture(torch, step_rm, 1)
    time_graphs(torch, graphs_rm, 3)
    per_rm = time_graphs(torch, graphs_rm, max(3, args.prefill_steps // 3)) / max(3, args.prefill_steps // 3)
    del graphs_rm
    flops = 6.0 * cfg.H * cfg.I * T * k
    touched = int((torch.diff(off) > 0).sum().item())
    wbytes = touched * cfg.expert_bytes
    binding = max(flops / PEAK_MXFP4, wbytes / PEAK_HBM)  # seconds at the binding roofline
    log(f"prefill4096: {per * 1e3:.3f} ms/layer, {T / per / 1e6:.2f} M tok/s, {touched} experts, "
        f"{wbytes / per / 1e9:.0f} GB/s of expert weights (row-major store: {per_rm * 1e3:.3f} ms; "
        f"packing the copy: {pack_ms:.1f} ms once)")
    log(f"prefill4096: per replay median {replays['median_us'] / 1e3:.3f} min {replays['min_us'] / 1e3:.3f} ms; "
        f"cold median {cold['median_us'] / 1e3:.3f} ms; sclk {clock_before['probe_sclk_mhz_median']:.0f} -> "
        f"{clock_after['probe_sclk_mhz_median']:.0f} MHz")
    return dict(ms_per_layer=per * 1e3, tokens_per_s=T / per, tflops=flops / per / 1e12,
                frac_of_mxfp4_peak=flops / per / PEAK_MXFP4,
                experts_touched=touched, weight_bytes=wbytes,
                weight_GBps=wbytes / per / 1e9, frac_of_peak_hbm_weights=wbytes / per / PEAK_HBM,
                frac_of_binding_roofline=binding / per, frac_of_measured_mfma=flops / per / MFMA_MEASURED,
                replays=replays, cold=dict(cold, flush_bytes=FLUSH_BYTES),
                clocks=dict(before=clock_before, after=clock_after),
                weights="operand-order copy for the tiled GEMMs (moe_ffn_fp4_prefill_packed)",
                pack_ms=pack_ms, packed_bytes=packed.numel(), row_major_ms_per_layer=per_rm * 1e3,
                mfma_busy=profile_fields(MFMA_FILE, PREFILL_SRC, ("gateup_tile_busy", "down_tile_busy",
                                                                  "gateup_skinny_busy", "down_skinny_busy")),
                _dev=dict(x=x, logits=logits, ids=ids, out=out))


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

    clk = Clock(torch, gd)
    clock_before = clk.read()
    graphs = capture(torch, token, 1)
    time_graphs(torch, graphs, 3)
    t = time_graphs(torch, graphs, args.chain_steps)
    per = t / args.chain_steps
    replays = stats_us(replay_series(torch, graphs[0], 1, REPLAYS))
    clock_after = clk.read()
    idn = ids.cpu().numpy()
    nbytes = sum(layer_bytes(cfg, len(set(idn[layer].reshape(-1).tolist())), T) + T * H * 2 * 2
                 for layer in range(cfg.layers))
    fin = xs[-1].float()
    finite = bool(torch.isfinite(fin).all().item())
    log(f"chain40: {per * 1e3:.3f} ms/token, {nbytes / per / 1e9:.0f} GB/s, finite={finite}")
    return dict(ms_per_token=per * 1e3, tokens_per_s=1.0 / per, gbps=nbytes / per / 1e9,
                frac_of_peak_hbm=nbytes / per / PEAK_HBM, bytes_per_token=nbytes, output_finite=finite,
                replays=replays, clocks=dict(before=clock_before, after=clock_after))


def cpu_baseline(db, gi, prefill=None) -> dict:
    """The fp64 numpy oracle timed on bounded samples of the workloads, on the
    host's cores: decode1 tokens with every BLAS thread and with one, one
    verify16 step, two tokens of the prefill4096 chunk (MXFP6 activations, the
    prefill reference), and one layer of the 40-layer chain.  Generating the
    weights is outside every timed region.  For the prefill tokens the GPU
    layer's output rows are compared with the oracle's (the prefill reference
    and the unquantised definition)."""
    import numpy as np
    from oracle import moe_oracle as o
    from threadpoolctl import threadpool_info, threadpool_limits
    blas = max([p_.get("num_threads", 1) for p_ in threadpool_info()] + [1])
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = nproc
    arms = {}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    # C1: decode1, one token per call
    cfg = db.cfg
    hw = gi.HostWeights(cfg)
    for name, n_tok, limit in (("decode1_all_threads", 4, None), ("decode1_one_thread", 3, 1)):
        tot_t, tot_b = 0.0, 0
        for i in range(n_tok):
            s_ = 8 + i if limit else i
            ids, _ = o.route(db.logit_sets[s_], cfg.k)
            for e in set(ids.reshape(-1).tolist()):
                for mat in range(3):
                    hw.matrix(int(e), mat)
            if limit:
                with threadpool_limits(limit):
                    _, dt = timed(lambda: o.moe_layer(db.hi.x_bf16, db.logit_sets[s_], hw.matrix, cfg.k, cfg.H))
            else:
                _, dt = timed(lambda: o.moe_layer(db.hi.x_bf16, db.logit_sets[s_], hw.matrix, cfg.k, cfg.H))
            tot_t += dt
            tot_b += layer_bytes(cfg, len(set(ids.reshape(-1).tolist())), cfg.T)
            hw.drop()
        arms[name] = dict(tokens=n_tok, seconds=round(tot_t, 2), GBps=round(tot_b / tot_t / 1e9, 4),
                          tokens_per_s=round(n_tok / tot_t, 3), blas_threads=limit or blas,
                          logit_sets=f"{8 if limit else 0}-{(8 if limit else 0) + n_tok - 1}")
    # C2: one verify16 step (16 tokens, Zipf-biased routing)
    c16 = gi.CONFIGS["verify16"]
    hi16 = gi.host_inputs(c16)
    lg16 = gi.logit_sets(c16, hi16.bias, 1)[0]
    ids16, _ = o.route(lg16, c16.k)
    hw16 = gi.HostWeights(c16)
    for e in set(ids16.reshape(-1).tolist()):
        for mat in range(3):
            hw16.matrix(int(e), mat)
    _, dt = timed(lambda: o.moe_layer(hi16.x_bf16, lg16, hw16.matrix, c16.k, c16.H))
    hw16.drop()
    arms["verify16_step"] = dict(tokens=c16.T, seconds=round(dt, 2), tokens_per_s=round(c16.T / dt, 3),
                                 experts=len(set(ids16.reshape(-1).tolist())), blas_threads=blas)
    # C4: two tokens of the prefill chunk through the prefill reference
    if prefill is not None:
        cp = gi.CONFIGS["prefill4096"]
        hip_ = gi.host_inputs(cp)
        toks = [0, cp.T // 2]
        x_s, lg_s = hip_.x_bf16[toks], hip_.logits[0][toks]
        idsp, _ = o.route(lg_s, cp.k)
        hwp = gi.HostWeights(cp)
        for e in set(idsp.reshape(-1).tolist()):
            for mat in range(3):
                hwp.matrix(int(e), mat)
        ref, dt = timed(lambda: o.moe_layer(x_s, lg_s, hwp.matrix, cp.k, cp.H, mode="a6"))
        ref16 = o.moe_layer(x_s, lg_s, hwp.matrix, cp.k, cp.H, mode="a16")
        hwp.drop()
        dev = prefill["_dev"]
        gpu_ids = dev["ids"][toks].cpu().numpy()
        gpu_out = dev["out"][toks].float().cpu().numpy().astype(np.float64)  # bf16 -> fp32 is exact
        scale = np.max(np.abs(ref["out"]))
        arms["prefill4096_sample"] = dict(
            tokens=len(toks), token_ids=toks, seconds=round(dt, 2), tokens_per_s=round(len(toks) / dt, 3),
            blas_threads=blas, gpu_ids_equal=bool(np.array_equal(gpu_ids, ref["ids"])),
            gpu_out_rel_vs_prefill_reference=float(np.max(np.abs(gpu_out - ref["out"])) / scale),
            gpu_out_rel_vs_unquantised=float(np.max(np.abs(gpu_out - ref16["out"])) / np.max(np.abs(ref16["out"]))))
    # C5: the first layer of the 40-layer chain (154 of 384 experts resident)
    c40 = gi.CONFIGS["chain40"]
    hi40 = gi.host_inputs(c40)
    hw40 = gi.HostWeights(c40, 0)
    e2s = hi40.expert_to_slot[0]
    ids40, _ = o.route(hi40.logits[0], c40.k, e2s)
    for e in set(ids40.reshape(-1).tolist()):
        if e2s[e] >= 0:
            for mat in range(3):
                hw40.matrix(int(e), mat)
    _, dt = timed(lambda: o.chain_layer(hi40.x_bf16, hi40.logits[0], hw40.matrix, c40.k, c40.H, e2s))
    hw40.drop()
    arms["chain40_one_layer"] = dict(layers=1, seconds=round(dt, 2), blas_threads=blas,
                                     ms_per_token_40_layers=round(40 * dt * 1e3, 1))
    head = arms["decode1_all_threads"]
    total = sum(a_["seconds"] for a_ in arms.values())
    log(f"cpu oracle: {total:.1f} s over {len(arms)} arms; decode1 {head['tokens_per_s']:.2f} tok/s "
        f"({head['GBps']:.3f} GB/s), one thread {arms['decode1_one_thread']['tokens_per_s']:.2f} tok/s")
    return dict(value=head["GBps"], unit="GB/s", cores=int(blas), kind="oracle",
                sample=f"decode1: {head['tokens']} single-token layers (logit sets {head['logit_sets']}) of the "
                       f"same workload, fp64 numpy oracle, weight generation excluded; numpy's elementwise work "
                       f"runs on one thread, only the matrix products use the {blas} BLAS threads",
                nproc=nproc, affinity_cpus=affinity, tokens_per_s=head["tokens_per_s"], arms=arms,
                seconds_total=round(total, 1))


def calibrate(torch, gd) -> dict:
    """Two kernels of known traffic that the HBM byte counters are scaled by:
    a plain device copy of 4 GiB (torch's copy kernel: 4 GiB read and 4 GiB
    written) and the streaming-read probe over 4 GiB (4 GiB read, nothing
    written).  Both are also measured streaming ceilings."""
    probe = read_ceiling(torch, gd)
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
    res = dict(copy=dict(bytes_read=n, bytes_written=n, us=t * 1e6, copy_GBps=2 * n / t / 1e9),
               read_probe=dict(bytes_read=probe["bytes"], bytes_written=0, us=probe["us"],
                               read_GBps=probe["read_GBps"]))
    log(f"calibration copy: {t * 1e6:.0f} us per 4 GiB copy, {2 * n / t / 1e9:.0f} GB/s read+write")
    return res


def load_probe(torch, gd) -> dict:
    """Per-CU rate of the shapes a weight tile can be loaded with (8 rows x 128
    B per load with the lanes along a row or across rows, 32 rows x 32 B (the
    MFMA operand order of a 32-row fragment), and the 8-row shapes copied into
    LDS by the buffer unit) against where the rows live: each XCD's 32
    workgroups stream 512-row sets of their own region of 1.3 MB (stays in the
    XCD's L2), 16.8 MB (memory-side cache) or 134 MB (HBM), with 4 or 8
    wavefronts of 32 KiB of loads in flight each (the LDS copies: 128 KiB per
    workgroup).  HIP events on the stream the probe runs on."""
    regions = (512, 6554, 52429)  # rows of 2560 B per XCD
    buf = torch.ones(8 * regions[-1] * 2560, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = gd.lib()
    stream = torch.cuda.current_stream()
    iters = 400
    rows = []
    for rr in regions:
        for waves in (4, 8):
            for pat in (0, 1, 2, 3, 4, 5, 6, 7, 8):
                def run():
                    assert L.gen_load_probe(buf.data_ptr(), rr, pat, waves, iters, sink.data_ptr(),
                                            stream.cuda_stream) == 0
                run()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 3
                e0.record(stream)
                for _ in range(reps):
                    run()
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) / 1e3 / reps
                nbytes = 256 * iters * 1024 * (128 if 3 <= pat <= 5 else 64 if pat == 7 else
                                               waves * 8 if pat == 8 else waves * 32)
                shape = ("8 rows x 128 B, lanes along rows", "32 rows x 32 B (MFMA order)",
                         "8 rows x 128 B, lanes across rows", "8 rows x 128 B across rows, into LDS",
                         "8 rows x 128 B along rows, into LDS", "8 rows along rows rotated, into LDS",
                         "8 rows along rows rotated", "8 rows rotated, into LDS, half in flight",
                         "8 rows x 128 B, 8 loads in flight")[pat]
                row = dict(region_MB_per_xcd=round(rr * 2560 / 1e6, 1), waves_per_cu=waves, shape=shape,
                           us=round(t * 1e6, 1), TBps=round(nbytes / t / 1e12, 2),
                           GBps_per_cu=round(nbytes / t / 1e9 / 256, 1))
                log(f"load probe: {row['region_MB_per_xcd']:6.1f} MB per XCD, {waves} waves/CU, "
                    f"{row['shape']:38s} {row['GBps_per_cu']:6.1f} GB/s per CU ({row['TBps']:.2f} TB/s)")
                rows.append(row)
    del buf
    torch.cuda.empty_cache()
    return dict(rows=rows)


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; --gpus must be 1"}))
        print("bench.py: only --gpus 1 is supported (the path is built and measured on one GPU)",
              file=sys.stderr)
        return 2
    prov = provenance()  # before the GPU is touched: the git query is a child process
    import torch
    import fp4_routed_expert_mxfp4_amd as m
    from gen import device as gd
    from gen import inputs as gi
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    prov.update(torch=torch.__version__, hip=torch.version.hip, device=torch.cuda.get_device_name(0))
    m.lib()
    if args.calibrate:
        print(json.dumps({"calibration": calibrate(torch, gd)}), flush=True)
        return 0
    if args.load_probe:
        res = load_probe(torch, gd)
        res["stream_read"] = read_ceiling(torch, gd)
        res["stream_read_lds"] = read_ceiling(torch, gd, lds=True)
        print(json.dumps({"load_probe": res}), flush=True)
        return 0

    if args.only:
        fn = {"decode": decode_section, "prefill": prefill_section, "chain": chain_section,
              "verify": verify_section, "router": router_gate_section, "cb3": cb3_section}[args.only]
        res = fn(args, torch, m, gd, gi)
        if isinstance(res, dict):
            res.pop("db", None)
            res.pop("_dev", None)
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
    cpu = None if args.no_cpu_baseline else cpu_baseline(dec["db"], gi, prefill)
    if prefill is not None:
        prefill.pop("_dev", None)

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
        "dtype": "mxfp4 (e2m1 codes, ue8m0 per 32) x bf16, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": "decode1: single-layer MoE FFN decode, batch 1, hidden 5120, expert width 2304, "
                               "384 MXFP4 experts resident, top-8, 64 rotating routings",
                   "hidden": cfg.H, "expert_width": cfg.I, "experts": cfg.E, "top_k": cfg.k, "tokens": cfg.T,
                   "weights": "e2m1 + UE8M0/32", "activations": "bf16"},
        "frac_of_peak_hbm": round(dec["gbps"] * 1e9 / PEAK_HBM, 4),
        "timing": {"value": f"one graph of {args.steps} back-to-back steps after {args.warmup} untimed ones, HIP "
                            "events on the replay stream",
                   "replays": dec["replays"], "cold_llc_flushed": dec["cold"],
                   "interleaved_medians": dec["interleaved"], "gateup_replays": dec["gateup_replays"],
                   "clocks": dec["clocks"]},
        "provenance": prov,
        "separate_calls_us_per_step": round(dec["separate_us"], 2),
        "batch_invariant_separate_calls_us_per_step": round(dec["invariant_us"], 2),
        "batch_invariant_layer_us_per_step": round(dec["invariant_layer_us"], 2),
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
