"""GPU parity of the prefill path (MXFP6 activations on block-scaled MFMA)
against the fp64 oracle's prefill reading, through the C ABI."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import PREFILL_A16_BOUND, REL_TOL, W_TOL, GpuLayer, bf16_excess, rel_err, to_np

pytestmark = pytest.mark.gpu

PREFILL_CASES = {
    "tiny": gi.CONFIGS["tiny"],
    # several row tiles per bucket (top bucket > 128 rows), ragged last tile, multi n-tiles
    "mid_zipf": gi.custom("mid_zipf_p", 1024, 384, 24, 4, 300, seed=31, zipf=1.1),
    # masked routable subset, k = 6
    "mid_resident": gi.custom("mid_resident_p", 512, 256, 40, 6, 77, seed=32, resident=10),
    # hidden 6144: the gate/up K loop spans two scale windows; buckets of ~100 rows (tiled path)
    "wide_hidden": gi.custom("wide_hidden_p", 6144, 256, 4, 2, 200, seed=33),
    # fewer routable experts (3) than k (4): weight-0 slots with zero rows
    "few_resident": gi.custom("few_resident_p", 512, 256, 16, 4, 9, seed=34, resident=3),
}


def pack6(codes: np.ndarray) -> np.ndarray:
    """e2m3 codes [rows][K] -> bytes [rows][K/32*24], code i of a block at bits 6i..6i+5."""
    rows, K = codes.shape
    c = codes.reshape(rows, K // 32, 32).astype(np.uint64)
    out = np.zeros((rows, K // 32, 3), dtype=np.uint64)
    for i in range(32):
        bit = 6 * i
        out[:, :, bit // 64] |= c[:, :, i] << np.uint64(bit % 64)
        if bit % 64 > 58:
            out[:, :, bit // 64 + 1] |= c[:, :, i] >> np.uint64(64 - bit % 64)
    return out.view(np.uint8).reshape(rows, K // 32 * 24)


def _oracle(gl: GpuLayer):
    c = gl.cfg
    return o.moe_layer(gl.hi.x_bf16, gl.hi.logits[gl.layer], gl.weights.matrix, c.k, c.H, "a6", gl.e2s_np)


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_layer_matches_oracle(name):
    print(f"case {name}", flush=True)
    gl = GpuLayer(PREFILL_CASES[name])
    r = gl.run("prefill")
    ref = _oracle(gl)
    np.testing.assert_array_equal(to_np(r["ids"]), ref["ids"])
    np.testing.assert_array_equal(to_np(r["sorted_pair"]), ref["sorted_pair"])
    assert np.max(np.abs(to_np(r["w"]) - ref["w"])) <= W_TOL
    e_y = rel_err(to_np(r["y_pair"]), ref["y_pair"])
    e_32 = rel_err(to_np(r["out32"]), ref["out"])
    e_16 = bf16_excess(to_np(r["out16"]), ref["out"])
    a16 = o.moe_layer(gl.hi.x_bf16, gl.hi.logits[0], gl.weights.matrix, gl.cfg.k, gl.cfg.H, "a16", gl.e2s_np)
    e_a16 = rel_err(to_np(r["out32"]), a16["out"])
    print(f"[{name}] y_pair rel {e_y:.3e}  out fp32 rel {e_32:.3e}  bf16 excess {e_16:.3e}  "
          f"distance to the unquantised (a16) definition {e_a16:.3e} (bound {PREFILL_A16_BOUND})", flush=True)
    assert e_y <= REL_TOL and e_32 <= REL_TOL and e_16 <= REL_TOL
    assert e_a16 <= PREFILL_A16_BOUND


def test_prefill_quantiser_bit_exact_all_bf16():
    """The x quantiser (first stage of the prefill call) against the oracle's
    Q6 on every finite bf16 value, read back from the workspace layout: codes
    [H/128][2][T*k][48 B] at offset 0 (per 128-K chunk c and K-half h, each
    sorted row's blocks 4c+h then 4c+2+h, 24 B each), then scale words
    [H/128][T*k] (the bytes of blocks 4c..4c+3).  With k = 1 and one expert
    the sorted rows are the tokens in order."""
    import fp4_routed_expert_mxfp4_amd as m
    H = 256
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).astype(np.uint32).view(np.float32)
    keep = np.isfinite(vals)
    xb = bits[keep].astype(np.uint16)
    T = len(xb) // H
    xb = xb[:T * H].reshape(T, H)
    cfg = gi.custom("q6all", H, 128, 8, 1, T, seed=5)
    gl = GpuLayer(cfg)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    ids = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    off, sp, _ = m.moe_permute(ids, cfg.E)
    np.testing.assert_array_equal(to_np(sp), np.arange(T))
    ws = torch.empty(m.prefill_workspace_bytes(T, 1, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    m.moe_ffn_fp4_prefill(x, 1, cfg.E, gl.store, None, off, sp, ws=ws)
    torch.cuda.synchronize()
    wsn = ws.cpu().numpy()
    nch = H // 128
    nq = T * H // 32 * 24
    rec = wsn[:nq].reshape(nch, 2, T, 48)
    blocks = np.empty((T, H // 32, 24), np.uint8)
    for bb in range(4):  # block 4c + bb: record of K-half bb % 2, bytes 24 (bb // 2) ..
        blocks[:, bb::4, :] = rec[:, bb % 2, :, 24 * (bb // 2):24 * (bb // 2) + 24].transpose(1, 0, 2)
    xq = blocks.reshape(T, H // 32 * 24)
    xs_off = (nq + 255) // 256 * 256
    xs = wsn[xs_off:xs_off + T * H // 32].reshape(nch, T, 4).transpose(1, 0, 2).reshape(T, H // 32)
    codes, sb = o.q6_rows(o.bf16_bits_to_f64(xb))
    np.testing.assert_array_equal(xs, sb)
    np.testing.assert_array_equal(xq, pack6(codes))


@pytest.fixture(scope="module")
def full_prefill():
    """The 4096-token chunk run once through route -> permute -> prefill FFN ->
    combine, in the launch configuration the benchmark times."""
    cfg = gi.CONFIGS["prefill4096"]
    print("case prefill4096 (full chunk)", flush=True)
    gl = GpuLayer(cfg)
    r = gl.run("prefill")
    ids_ref, w_ref = o.route(gl.hi.logits[0], cfg.k)
    np.testing.assert_array_equal(to_np(r["ids"]), ids_ref)
    offsets = to_np(r["offsets"])
    sp = to_np(r["sorted_pair"])
    yield dict(cfg=cfg, gl=gl, r=r, ids=ids_ref, w=w_ref, offsets=offsets, sp=sp)
    gl.weights.drop()


def _stratified_rows(offsets):
    """Rows of every touched expert's bucket to compare: all of a bucket of at
    most 48 rows (the small-bucket streaming kernels take up to 32), else its
    first 8 rows, its last 160 (the ragged last row tile and the full tile
    before it, for row tiles of up to 160) and every 97th row between."""
    plan = []
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        n = b - a
        if n == 0:
            continue
        if n <= 48:
            rows = list(range(n))
        else:
            rows = sorted(set(range(8)) | set(range(max(0, n - 160), n)) | set(range(0, n, 97)))
        plan.append((e, [a + r for r in rows]))
    return plan


N_PARTS = 4


@pytest.mark.parametrize("part", range(N_PARTS))
def test_prefill_full_size_every_expert(full_prefill, part):
    """Every touched expert of the 4096-token chunk has rows compared with the
    oracle: every row of the small buckets, and the first rows, the ragged
    last tile and a spread of rows of every tiled bucket.  The experts are
    split over N_PARTS tests (round robin) to keep each under a minute."""
    f = full_prefill
    cfg, gl = f["cfg"], f["gl"]
    plan = _stratified_rows(f["offsets"])[part::N_PARTS]
    if part == 0:
        sizes = np.diff(f["offsets"])
        print(f"prefill4096: {np.count_nonzero(sizes)} experts touched, {np.count_nonzero((sizes > 0) & (sizes <= 32))} "
              f"small buckets, largest {sizes.max()} rows", flush=True)
    worst, nrows = 0.0, 0
    for e, rows in plan:
        pairs = f["sp"][rows]
        y_dev = f["r"]["y_pair"][torch.from_numpy(pairs.astype(np.int64)).cuda()]
        x = o.bf16_bits_to_f64(gl.hi.x_bf16[pairs // cfg.k])
        y_ref = o.expert_ffn(x, gl.weights.matrix, e, "a6")
        err = rel_err(to_np(y_dev), y_ref)
        worst = max(worst, err)
        nrows += len(rows)
        gl.weights.drop()
        assert err <= REL_TOL, f"expert {e}: rel {err:.3e} over {len(rows)} rows"
    print(f"[prefill4096 part {part}] {len(plan)} experts, {nrows} rows, worst expert rel {worst:.3e}", flush=True)


def test_prefill_full_size_sampled_tokens(full_prefill):
    """Whole tokens of the 4096-token chunk (all k rows and the combine) on a
    sample the oracle evaluates one by one; byte determinism of a rerun."""
    f = full_prefill
    cfg, gl, r = f["cfg"], f["gl"], f["r"]
    rng = np.random.default_rng(0)
    sample = sorted(set([0, cfg.T - 1] + list(rng.choice(cfg.T, 6, replace=False))))
    x = gl.hi.x_bf16[sample]
    y_ref = o.ffn(x, f["ids"][sample], gl.weights.matrix, cfg.H, "a6")
    gl.weights.drop()
    out_ref = o.combine(y_ref, f["w"][sample])
    y = to_np(r["y_pair"]).reshape(cfg.T, cfg.k, cfg.H)[sample].reshape(-1, cfg.H)
    e_y = rel_err(y, y_ref)
    e_32 = rel_err(to_np(r["out32"])[sample], out_ref)
    e_16 = bf16_excess(to_np(r["out16"])[sample], out_ref)
    print(f"[prefill4096, {len(sample)} tokens] y_pair rel {e_y:.3e} out fp32 rel {e_32:.3e} bf16 excess {e_16:.3e}")
    assert e_y <= REL_TOL and e_32 <= REL_TOL and e_16 <= REL_TOL
    # every output row finite, and the run is byte-deterministic
    assert np.isfinite(to_np(r["out32"])).all()
    r2 = gl.run("prefill")
    assert torch.equal(r["y_pair"], r2["y_pair"]) and torch.equal(r["out16"], r2["out16"])


@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_out_of_range_ids_are_left_out(path):
    """Pairs whose expert id lies outside [0, E) are in no bucket: the FFN
    reads no row of them and writes no y_pair row for them (the rows keep what
    they held), and every other row equals the oracle's.  route -> permute ->
    FFN -> combine, with the ids edited between route and permute."""
    import fp4_routed_expert_mxfp4_amd as m
    cfg = gi.custom(f"badids_{path}", 512, 256, 16, 4, 40, seed=35)
    print(f"case badids {path}", flush=True)
    gl = GpuLayer(cfg)
    ids_ref, w_ref = o.route(gl.hi.logits[0], cfg.k)
    ids = ids_ref.copy()
    bad = [(3, 1, -1), (7, 0, cfg.E), (20, 3, -5), (39, 2, 1 << 20)]
    for t, j, v in bad:
        ids[t, j] = v
    dev_ids = torch.from_numpy(ids).cuda()
    off, sp, p2r = m.moe_permute(dev_ids, cfg.E)
    offn = to_np(off)
    assert offn[-1] == cfg.T * cfg.k - len(bad)
    p2rn = to_np(p2r)
    for t, j, _ in bad:
        assert p2rn[t * cfg.k + j] == -1
    sentinel = 12345.0
    y = torch.full((cfg.T * cfg.k, cfg.H), sentinel, dtype=torch.float32, device="cuda")
    ffn = m.moe_ffn_fp4_prefill if path == "prefill" else m.moe_ffn_fp4_decode
    ffn(gl.x, cfg.k, cfg.E, gl.store, None, off, sp, y_pair=y)
    torch.cuda.synchronize()
    yn = to_np(y)
    mode = "a6" if path == "prefill" else "a16"
    ok = np.ones(cfg.T * cfg.k, bool)
    for t, j, _ in bad:
        ok[t * cfg.k + j] = False
        assert np.all(yn[t * cfg.k + j] == sentinel)
    y_ref = o.ffn(gl.hi.x_bf16, np.where(ids_ref >= 0, ids_ref, 0), gl.weights.matrix, cfg.H, mode)
    e = rel_err(yn[ok], y_ref[ok])
    # the combine of the tokens without an out-of-range id matches the oracle's
    w_dev = torch.from_numpy(w_ref.astype(np.float32)).cuda()
    out = to_np(m.moe_combine(y, w_dev, None, m.MOE_OUT_F32))
    good_t = sorted(set(range(cfg.T)) - {t for t, _, _ in bad})
    e_out = rel_err(out[good_t], o.combine(y_ref, w_ref)[good_t])
    print(f"[badids {path}] valid rows rel {e:.3e}, combined rel {e_out:.3e}", flush=True)
    assert e <= REL_TOL and e_out <= REL_TOL
