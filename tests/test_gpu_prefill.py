"""GPU parity of the prefill path (MXFP6 activations on block-scaled MFMA)
against the fp64 oracle's prefill reading, through the C ABI."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, W_TOL, GpuLayer, bf16_excess, rel_err, to_np

pytestmark = pytest.mark.gpu

PREFILL_CASES = {
    "tiny": gi.CONFIGS["tiny"],
    # several row tiles per bucket (top bucket > 128 rows), ragged last tile, multi n-tiles
    "mid_zipf": gi.custom("mid_zipf_p", 1024, 384, 24, 4, 300, seed=31, zipf=1.1),
    # masked routable subset, k = 6
    "mid_resident": gi.custom("mid_resident_p", 512, 256, 40, 6, 77, seed=32, resident=10),
    # hidden 6144: the gate/up K loop spans two scale windows; buckets of ~100 rows (tiled path)
    "wide_hidden": gi.custom("wide_hidden_p", 6144, 256, 4, 2, 200, seed=33),
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
    e_info = rel_err(to_np(r["out32"]), a16["out"])
    print(f"[{name}] y_pair rel {e_y:.3e}  out fp32 rel {e_32:.3e}  bf16 excess {e_16:.3e}  "
          f"(vs unquantised reference, for information: {e_info:.3e})", flush=True)
    assert e_y <= REL_TOL and e_32 <= REL_TOL and e_16 <= REL_TOL


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


def test_prefill_full_size_sampled_tokens():
    """The 4096-token chunk in the launch configuration the benchmark times,
    checked on a sample of tokens the oracle evaluates one by one."""
    cfg = gi.CONFIGS["prefill4096"]
    gl = GpuLayer(cfg)
    r = gl.run("prefill")
    ids_ref, w_ref = o.route(gl.hi.logits[0], cfg.k)
    np.testing.assert_array_equal(to_np(r["ids"]), ids_ref)
    # sample: tokens whose experts are few and shared, plus the first and last token
    rng = np.random.default_rng(0)
    pop = np.bincount(ids_ref.reshape(-1), minlength=cfg.E)
    top = set(np.argsort(-pop)[:24].tolist())
    cands = [t for t in range(cfg.T) if sum(int(e) in top for e in ids_ref[t]) >= 7]
    sample = sorted(set([0, cfg.T - 1] + list(rng.choice(cands, 10, replace=False))))
    x = gl.hi.x_bf16[sample]
    y_ref = o.ffn(x, ids_ref[sample], gl.weights.matrix, cfg.H, "a6")
    out_ref = o.combine(y_ref, w_ref[sample])
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
