"""moe_decode_layer_noalloc (the library's static scratch, no workspace
argument) against moe_decode_layer with a caller workspace: the same kernels,
so every output must be bit-identical.  Two calls in a row on the same GPU,
the second with a smaller input, then a request beyond the scratch's size."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from tests.harness import GpuLayer, to_np

pytestmark = pytest.mark.gpu


def _both(m, gl, logits, x, residual, od):
    k = gl.cfg.k
    ref = m.moe_decode_layer(logits, x, k, gl.store, gl.e2s, residual, od)
    got = m.moe_decode_layer_noalloc(logits, x, k, gl.store, gl.e2s, residual, od)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_layer_equals_workspace_layer():
    import fp4_routed_expert_mxfp4_amd as m
    # first call: 16 tokens (route, bucketing, multi-token FFN, combine through the scratch)
    cfg16 = gi.CONFIGS["verify16"]
    print("case noalloc verify16", flush=True)
    gl = GpuLayer(cfg16)
    for od in (m.MOE_OUT_BF16, m.MOE_OUT_F32):
        ref, got = _both(m, gl, gl.logits, gl.x, gl.x, od)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    del gl
    torch.cuda.empty_cache()
    # second call, smaller input: one token (the two fused kernels), the scratch keeps the last call's bytes
    cfg1 = gi.CONFIGS["decode1"]
    print("case noalloc decode1", flush=True)
    gl = GpuLayer(cfg1)
    sets = gi.logit_sets(cfg1, gl.hi.bias, 2)
    for i in range(2):
        logits = torch.from_numpy(sets[i]).cuda()
        ref, got = _both(m, gl, logits, gl.x, None, m.MOE_OUT_BF16)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        assert np.isfinite(to_np(got[2])).all()


def test_noalloc_rejects_beyond_scratch():
    import fp4_routed_expert_mxfp4_amd as m
    # 256 tokens at the full shape need 58 MiB of workspace, past the 32 MiB scratch
    T, E, k, H, I = 256, 384, 8, 5120, 2304
    assert m.decode_layer_workspace_bytes(T, k, E, H, I) > m.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    z = lambda *shape: torch.zeros(shape, dtype=torch.uint8, device=dev)
    store = m.ExpertStore(z(1, I, H // 2), z(1, I, H // 32), z(1, I, H // 2), z(1, I, H // 32),
                          z(1, H, I // 2), z(1, H, I // 32))
    e2s = torch.full((E,), -1, dtype=torch.int32, device=dev)
    e2s[:8] = 0
    logits = torch.zeros((T, E), dtype=torch.float32, device=dev)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    with pytest.raises(m.MoeError) as ei:
        m.moe_decode_layer_noalloc(logits, x, k, store, e2s)
    assert ei.value.status == 5  # MOE_ERR_WORKSPACE
