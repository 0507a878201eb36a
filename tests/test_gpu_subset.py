"""The expert-subset FFN calls (the two-wave routed MoE: experts on hand now,
the rest once they arrive), through the C ABI.  Two calls whose run masks
cover every expert once leave y_pair bit-identical to one call over all
experts, and a call leaves the rows of the experts outside its mask exactly as
they were."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, GpuLayer, rel_err, to_np

pytestmark = pytest.mark.gpu

CASES = {
    # one token at the one-token shape (VALU kernels)
    "decode1": ("decode", gi.CONFIGS["decode1"]),
    # 16 tokens (bf16 MFMA kernels)
    "verify16": ("decode", gi.CONFIGS["verify16"]),
    # masked routable subset: experts without a slot write zero rows when they run
    "mid_resident": ("decode", gi.custom("mid_resident", 768, 256, 40, 3, 9, seed=22, resident=12)),
    # prefill with small-bucket and tiled experts
    "prefill_mid_zipf": ("prefill", gi.custom("mid_zipf_p", 1024, 384, 24, 4, 300, seed=31, zipf=1.1)),
    "prefill_tiny": ("prefill", gi.CONFIGS["tiny"]),
}
SENTINEL = 12345.0


def _ffn(m, path, gl, off, sp, mask, y=None):
    c = gl.cfg
    if mask is None:
        f = m.moe_ffn_fp4_decode if path == "decode" else m.moe_ffn_fp4_prefill
        return f(gl.x, c.k, c.E, gl.store, gl.e2s, off, sp, y)
    f = m.moe_ffn_fp4_decode_subset if path == "decode" else m.moe_ffn_fp4_prefill_subset
    return f(gl.x, c.k, c.E, gl.store, gl.e2s, off, sp, mask, y)


def _setup(name):
    import fp4_routed_expert_mxfp4_amd as m
    path, cfg = CASES[name]
    print(f"case {name}", flush=True)
    gl = GpuLayer(cfg)
    ids, _ = m.moe_route(gl.logits, cfg.k, gl.e2s)
    off, sp, _ = m.moe_permute(ids, cfg.E)
    full = _ffn(m, path, gl, off, sp, None)
    torch.cuda.synchronize()
    return m, path, cfg, gl, off, sp, to_np(ids).reshape(-1), to_np(full)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("name", list(CASES))
def test_two_waves_equal_one_pass(name):
    m, path, cfg, gl, off, sp, pair_expert, full = _setup(name)
    on = np.random.default_rng(5).random(cfg.E) < 0.5  # a seeded half of the experts is on hand
    on[pair_expert[0]] = True                           # both waves have rows to write
    on[pair_expert[-1]] = pair_expert[-1] == pair_expert[0]
    y = torch.full((cfg.T * cfg.k, cfg.H), SENTINEL, dtype=torch.float32, device="cuda")
    first = on[pair_expert]
    _ffn(m, path, gl, off, sp, torch.from_numpy(on.astype(np.uint8)).cuda(), y)
    torch.cuda.synchronize()
    got = to_np(y)
    assert np.array_equal(_bits(got[first]), _bits(full[first]))
    assert np.all(got[~first] == SENTINEL)
    _ffn(m, path, gl, off, sp, torch.from_numpy((~on).astype(np.uint8)).cuda(), y)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(to_np(y)), _bits(full))


@pytest.mark.parametrize("name", ["mid_resident", "prefill_mid_zipf", "prefill_tiny"])
def test_first_wave_matches_oracle(name):
    """The rows one wave writes against the oracle's rows of the same pairs (decode: the
    unquantised reading; prefill: the MXFP6 reading)."""
    m, path, cfg, gl, off, sp, pair_expert, _ = _setup(name)
    on = np.zeros(cfg.E, dtype=bool)
    on[::3] = True
    on[pair_expert[0]] = True
    y = torch.full((cfg.T * cfg.k, cfg.H), SENTINEL, dtype=torch.float32, device="cuda")
    _ffn(m, path, gl, off, sp, torch.from_numpy(on.astype(np.uint8)).cuda(), y)
    torch.cuda.synchronize()
    ref = o.moe_layer(gl.hi.x_bf16, gl.hi.logits[gl.layer], gl.weights.matrix, cfg.k, cfg.H,
                      "a16" if path == "decode" else "a6", gl.e2s_np)["y_pair"]
    first = on[pair_expert]
    got = to_np(y)
    e = rel_err(got[first], ref[first])
    print(f"[{name}] {int(first.sum())} of {first.size} rows, rel {e:.3e}", flush=True)
    assert e <= REL_TOL
    assert np.all(got[~first] == SENTINEL)


@pytest.mark.parametrize("name", ["verify16", "prefill_tiny"])
def test_empty_and_full_masks(name):
    m, path, cfg, gl, off, sp, _, full = _setup(name)
    y = torch.full((cfg.T * cfg.k, cfg.H), SENTINEL, dtype=torch.float32, device="cuda")
    _ffn(m, path, gl, off, sp, torch.zeros(cfg.E, dtype=torch.uint8, device="cuda"), y)
    torch.cuda.synchronize()
    assert np.all(to_np(y) == SENTINEL)
    _ffn(m, path, gl, off, sp, torch.full((cfg.E,), 7, dtype=torch.uint8, device="cuda"), y)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(to_np(y)), _bits(full))
