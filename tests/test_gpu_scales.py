"""GPU parity with UE8M0 scale bytes spread far beyond the configs' range.

The synthetic configs draw scale exponents from [-6, 0] (bytes 121-127).
Here every scale byte of the expert store is redrawn: bytes 100-140 for most
blocks, 1-3 for about 2 % of them (values down to 2^-127 times an e2m1 code,
below the smallest normal bf16) and 145-150 for about 0.5 % (up to 2^23).
The largest bytes are chosen so that no exact result can leave the fp32
range: with |x| < 6 and every weight at most 6 * 2^23, |g|, |u| < 2e12,
|h| < 4e24 and |y| < 3e35 even with all terms aligned (bytes of 160 in all
three matrices can take y past 3.4e38, where the fp32 kernels rightly give
infinity and the fp64 oracle does not).
The one-token (VALU) decode kernels, the multi-token (bf16 MFMA) decode
kernels, the batch-invariant call and the prefill (MXFP6 x MXFP4 MFMA)
kernels are each compared with the fp64 oracle on the same bytes.  Byte 255
(NaN in the OCP MX encoding) is outside the accepted input range and is not
drawn.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, GpuLayer, rel_err, to_np

pytestmark = pytest.mark.gpu


def _wide_scales(gl: GpuLayer, seed: int):
    """Redraw every scale byte of the layer's store on the host (seeded) and
    upload them; returns the oracle's weights callback over the new bytes."""
    rng = np.random.default_rng(seed)
    host = {}
    for m, name in ((0, "s_gate"), (1, "s_up"), (2, "s_down")):
        t = getattr(gl.store, name)
        b = rng.integers(100, 141, size=tuple(t.shape)).astype(np.uint8)
        u = rng.random(b.shape)
        b[u < 0.02] = rng.integers(1, 4, size=int(np.count_nonzero(u < 0.02))).astype(np.uint8)
        hi = (u >= 0.02) & (u < 0.025)
        b[hi] = rng.integers(145, 151, size=int(np.count_nonzero(hi))).astype(np.uint8)
        t.copy_(torch.from_numpy(b))
        host[m] = b
    torch.cuda.synchronize()
    base = gl.weights.matrix
    slot = (lambda e: e) if gl.e2s_np is None else (lambda e: int(gl.e2s_np[e]))
    return lambda e, m: (base(e, m)[0], host[m][slot(e)])


CASES = {
    # one token at a one-token kernel shape (hidden 2048, width 2304: 72 blocks per down row)
    "one_token": (gi.custom("wide_scale_1", 2048, 2304, 16, 4, 1, seed=41), "decode"),
    # several tokens: the multi-token kernels
    "multi_token": (gi.custom("wide_scale_13", 1024, 384, 12, 4, 13, seed=42, zipf=1.1), "decode"),
    # the batch-invariant call (multi-token arithmetic for one token)
    "invariant": (gi.custom("wide_scale_inv", 2048, 2304, 16, 4, 1, seed=43), "invariant"),
    # prefill: tiled buckets (about 100 rows) and small ones
    "prefill": (gi.custom("wide_scale_p", 1024, 384, 6, 2, 300, seed=44, zipf=1.1), "prefill"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_wide_scale_bytes_match_oracle(name):
    import fp4_routed_expert_mxfp4_amd as m
    cfg, path = CASES[name]
    print(f"case {name}", flush=True)
    gl = GpuLayer(cfg)
    weights = _wide_scales(gl, 500 + len(name))
    ids, w = m.moe_route(gl.logits, cfg.k, gl.e2s)
    off, sp, _ = m.moe_permute(ids, cfg.E)
    call = {"decode": m.moe_ffn_fp4_decode, "invariant": m.moe_ffn_fp4_decode_invariant,
            "prefill": m.moe_ffn_fp4_prefill}[path]
    y = call(gl.x, cfg.k, cfg.E, gl.store, gl.e2s, off, sp)
    out = m.moe_combine(y, w, None, m.MOE_OUT_F32)
    torch.cuda.synchronize()
    mode = "a6" if path == "prefill" else "a16"
    ref = o.moe_layer(gl.hi.x_bf16, gl.hi.logits[0], weights, cfg.k, cfg.H, mode, gl.e2s_np)
    np.testing.assert_array_equal(to_np(ids), ref["ids"])
    yn = to_np(y)
    assert np.isfinite(yn).all()
    e_y = rel_err(yn, ref["y_pair"])
    e_out = rel_err(to_np(out), ref["out"])
    # row by row as well: the rows of small-scale experts are not hidden behind the large ones
    e_row = max(rel_err(yn[p], ref["y_pair"][p]) for p in range(yn.shape[0]) if np.any(ref["y_pair"][p]))
    print(f"[{name}] max|y| {np.max(np.abs(ref['y_pair'])):.3e}  y_pair rel {e_y:.3e}  worst row {e_row:.3e}  "
          f"out rel {e_out:.3e}", flush=True)
    assert e_y <= REL_TOL and e_out <= REL_TOL and e_row <= REL_TOL
