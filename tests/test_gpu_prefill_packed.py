"""The prefill FFN on the experts' copy in MFMA operand order
(moe_prefill_pack_weights, moe_ffn_fp4_prefill_packed: tiled and small-bucket
kernels both read the copy), through the C ABI:
the copy's layout against its definition in the header, and the packed call
bit-identical to moe_ffn_fp4_prefill (which the prefill parity tests compare
with the oracle), plus a direct oracle comparison."""
import numpy as np
import pytest
import torch

import fp4_routed_expert_mxfp4_amd as m
from gen import inputs as gi
from oracle import moe_oracle as o
from tests.harness import REL_TOL, GpuLayer, rel_err, to_np

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": gi.CONFIGS["tiny"],
    "mid_zipf": gi.custom("mid_zipf_p", 1024, 384, 24, 4, 300, seed=31, zipf=1.1),
    "mid_resident": gi.custom("mid_resident_p", 512, 256, 40, 6, 77, seed=32, resident=10),
    # inter % 256 == 128 (a half-empty last pair in down, a half-wide last gate/up tile) and
    # hidden % 512 == 256 (a half-wide last down tile); buckets of up to ~150 rows
    "ragged": gi.custom("ragged_pk", 768, 640, 6, 2, 300, seed=35, zipf=1.1),
    # two scale windows along hidden
    "wide_hidden": gi.custom("wide_hidden_p", 6144, 256, 4, 2, 200, seed=33),
}


def pack_reference(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One matrix [rows][K/2] codes, [rows][K/32] scales -> its packed blocks, as the header defines them."""
    rows, KB = codes.shape
    K = 2 * KB
    npairs = (K + 255) // 256
    out = np.zeros((rows // 32, npairs, 4352), dtype=np.uint8)
    c = np.zeros((rows, npairs * 128), dtype=np.uint8)
    c[:, :KB] = codes
    s = np.zeros((rows, npairs * 8), dtype=np.uint8)
    s[:, :K // 32] = scales
    for lane in range(64):
        r32, h = lane % 32, lane // 32
        rr = np.arange(rows // 32) * 32 + r32
        for S in range(4):
            for j in range(npairs):
                out[:, j, S * 1024 + 16 * lane:S * 1024 + 16 * lane + 16] = c[rr, 128 * j + 32 * S + 16 * h:
                                                                                  128 * j + 32 * S + 16 * h + 16]
        for j in range(npairs):
            for S in range(4):
                out[:, j, 4096 + 4 * lane + S] = s[rr, 8 * j + 2 * S + h]
    return out.reshape(-1)


def test_packed_layout_matches_its_definition():
    gl = GpuLayer(gi.custom("pack_layout", 512, 384, 3, 2, 4, seed=36))
    st = gl.store
    pk = m.moe_prefill_pack_weights(st)
    torch.cuda.synchronize()
    got = to_np(pk)
    assert got.size == m.prefill_packed_bytes(st.num_slots, st.hidden, st.inter)
    per_slot = got.size // st.num_slots
    for slot in range(st.num_slots):
        ref = np.concatenate([pack_reference(to_np(st.w_gate[slot]), to_np(st.s_gate[slot])),
                              pack_reference(to_np(st.w_up[slot]), to_np(st.s_up[slot])),
                              pack_reference(to_np(st.w_down[slot]), to_np(st.s_down[slot]))])
        np.testing.assert_array_equal(got[slot * per_slot:(slot + 1) * per_slot], ref)


def _both(gl: GpuLayer):
    cfg = gl.cfg
    ids, w = m.moe_route(gl.logits, cfg.k, gl.e2s)
    off, sp, _ = m.moe_permute(ids, cfg.E)
    y0 = m.moe_ffn_fp4_prefill(gl.x, cfg.k, cfg.E, gl.store, gl.e2s, off, sp)
    pk = m.moe_prefill_pack_weights(gl.store)
    y1 = torch.full_like(y0, float("nan"))
    m.moe_ffn_fp4_prefill_packed(gl.x, cfg.k, cfg.E, gl.store, pk, gl.e2s, off, sp, y_pair=y1)
    torch.cuda.synchronize()
    return ids, w, off, sp, y0, y1


@pytest.mark.parametrize("name", list(CASES))
def test_packed_prefill_bit_identical(name):
    print(f"case {name}", flush=True)
    gl = GpuLayer(CASES[name])
    ids, w, off, sp, y0, y1 = _both(gl)
    offn = to_np(off)
    sizes = np.diff(offn)
    print(f"[{name}] buckets over 32 rows: {int((sizes > 32).sum())}, largest {int(sizes.max())}", flush=True)
    valid = to_np(sp)[:int(offn[-1])]
    assert torch.equal(y0[valid], y1[valid])
    if name in ("ragged", "mid_zipf"):
        ref = o.moe_layer(gl.hi.x_bf16, gl.hi.logits[gl.layer], gl.weights.matrix, gl.cfg.k, gl.cfg.H, "a6",
                          gl.e2s_np)
        e = rel_err(to_np(y1), ref["y_pair"])
        print(f"[{name}] packed y_pair rel err against the oracle {e:.3e}", flush=True)
        assert e <= REL_TOL


def test_packed_prefill_full_chunk_bit_identical():
    """The 4096-token chunk (hidden 5120, width 2304, 384 experts, Zipf 1.1): every row."""
    print("case prefill4096", flush=True)
    gl = GpuLayer(gi.CONFIGS["prefill4096"])
    ids, w, off, sp, y0, y1 = _both(gl)
    valid = to_np(sp)[:int(to_np(off)[-1])]
    assert torch.equal(y0[valid], y1[valid])
