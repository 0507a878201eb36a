"""The C-ABI library loads without a GPU, exports every symbol the header
declares, and rejects bad arguments with status codes before touching HIP.
No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp4.h")


def _lib():
    from fp4_routed_expert_mxfp4_amd import moe
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe_fp4.so not built")
    return moe


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"MOE_FP4_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


def test_header_declares_the_five_calls():
    names = set(declared_functions())
    for n in ("moe_route", "moe_permute", "moe_ffn_fp4_decode", "moe_ffn_fp4_prefill", "moe_combine"):
        assert n in names


def test_library_exports_every_declared_symbol():
    m = _lib()
    L = ctypes.CDLL(m.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(m.EXPORTED)


def test_gen_library_exports():
    from gen import device as gd
    if not os.path.exists(gd.LIB_PATH):
        pytest.skip("libmoe_gen.so not built")
    L = ctypes.CDLL(gd.LIB_PATH)
    for name in ("gen_fill_codes", "gen_fill_scales", "gen_stream_read", "gen_stream_read_lds", "gen_clock_probe",
                 "gen_load_probe"):
        assert hasattr(L, name), name


def test_gen_load_probe_rejects_bad_arguments():
    """The weight-tile load probe refuses shapes it has no kernel for before
    touching the GPU (no launch happens on the CPU)."""
    from gen import device as gd
    if not os.path.exists(gd.LIB_PATH):
        pytest.skip("libmoe_gen.so not built")
    L = gd.lib()
    good = dict(region_rows=512, pattern=0, waves=4, iters=1)
    for bad in (dict(region_rows=511), dict(region_rows=1 << 20), dict(pattern=9), dict(pattern=-1), dict(waves=6),
                dict(iters=0)):
        a = dict(good, **bad)
        assert L.gen_load_probe(FAKE, a["region_rows"], a["pattern"], a["waves"], a["iters"], FAKE, None) == 1, bad
    assert L.gen_load_probe(None, 512, 0, 4, 1, FAKE, None) == 1


def test_status_strings():
    m = _lib()
    for s in range(7):
        assert m.status_string(s)
    assert m.status_string(99) == "unknown status"


FAKE = 0x10000          # a 256-aligned address that is never dereferenced by validation
MIS = 0x10001


def _store(m, **over):
    d = dict(num_slots=8, hidden=256, inter=128, w_gate=FAKE, s_gate=FAKE, w_up=FAKE, s_up=FAKE,
             w_down=FAKE, s_down=FAKE)
    d.update(over)
    return m.CExperts(d["num_slots"], d["hidden"], d["inter"], d["w_gate"], d["s_gate"], d["w_up"],
                      d["s_up"], d["w_down"], d["s_down"])


def test_route_validation():
    m = _lib()
    L = m.lib()
    assert L.moe_route(None, 1, 8, 2, None, FAKE, FAKE, None) == m.MOE_ERR_NULL
    assert L.moe_route(FAKE, 1, 8, 9, None, FAKE, FAKE, None) == m.MOE_ERR_SHAPE       # k > E
    assert L.moe_route(FAKE, 1, 8, 0, None, FAKE, FAKE, None) == m.MOE_ERR_SHAPE       # k = 0
    assert L.moe_route(FAKE, 1, 8, 17, None, FAKE, FAKE, None) == m.MOE_ERR_SHAPE      # k > 16
    assert L.moe_route(FAKE, 1, 1025, 2, None, FAKE, FAKE, None) == m.MOE_ERR_SHAPE    # E > 1024
    assert L.moe_route(FAKE, -1, 8, 2, None, FAKE, FAKE, None) == m.MOE_ERR_SHAPE
    assert L.moe_route(None, 0, 8, 2, None, None, None, None) == m.MOE_OK              # empty batch


def test_permute_validation():
    m = _lib()
    L = m.lib()
    assert L.moe_permute(FAKE, 1, 2, 8, None, FAKE, FAKE, None, 0, None) == m.MOE_ERR_NULL
    assert L.moe_permute(None, 1, 2, 8, FAKE, FAKE, FAKE, None, 0, None) == m.MOE_ERR_NULL
    assert L.moe_permute(FAKE, 1, 2, 2000, FAKE, FAKE, FAKE, None, 0, None) == m.MOE_ERR_SHAPE
    assert L.moe_permute(FAKE, 1 << 22, 8, 8, FAKE, FAKE, FAKE, None, 0, None) == m.MOE_ERR_SHAPE
    # more than one 1024-pair chunk needs the workspace
    need = m.permute_workspace_bytes(4096, 8, 384)
    assert need == 32 * 384 * 4
    assert m.permute_workspace_bytes(128, 8, 384) == 0
    assert L.moe_permute(FAKE, 4096, 8, 384, FAKE, FAKE, FAKE, None, 0, None) == m.MOE_ERR_WORKSPACE
    assert L.moe_permute(FAKE, 4096, 8, 384, FAKE, FAKE, FAKE, FAKE, need - 1, None) == m.MOE_ERR_WORKSPACE
    assert L.moe_permute(FAKE, 4096, 8, 384, FAKE, FAKE, FAKE, FAKE + 16, need, None) == m.MOE_ERR_ALIGN


def _decode(m, x=FAKE, T=1, k=2, E=8, store=None, e2s=None, off=FAKE, sp=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 20):
    st = _store(m) if store is None else store
    return m.lib().moe_ffn_fp4_decode(x, T, k, E, ctypes.byref(st), e2s, off, sp, y, ws, ws_bytes, None)


def test_decode_validation():
    m = _lib()
    assert _decode(m, x=None) == m.MOE_ERR_NULL
    assert _decode(m, store=_store(m, w_up=None)) == m.MOE_ERR_NULL
    assert _decode(m, store=_store(m, hidden=200)) == m.MOE_ERR_SHAPE
    assert _decode(m, store=_store(m, inter=100)) == m.MOE_ERR_SHAPE
    assert _decode(m, store=_store(m, hidden=32768)) == m.MOE_ERR_UNSUPPORTED
    assert _decode(m, store=_store(m, num_slots=4)) == m.MOE_ERR_SHAPE          # identity needs S >= E
    assert _decode(m, x=MIS) == m.MOE_ERR_ALIGN
    assert _decode(m, store=_store(m, w_down=MIS)) == m.MOE_ERR_ALIGN
    assert _decode(m, ws=None) == m.MOE_ERR_WORKSPACE
    assert _decode(m, ws_bytes=16) == m.MOE_ERR_WORKSPACE
    assert _decode(m, ws=FAKE + 16) == m.MOE_ERR_ALIGN
    assert _decode(m, T=300) == m.MOE_ERR_UNSUPPORTED
    assert _decode(m, k=9) == m.MOE_ERR_SHAPE
    assert _decode(m, T=0) == m.MOE_OK
    assert m.decode_workspace_bytes(1, 8, 2304) == 8 * 2304 * 4


def test_subset_validation():
    """The expert-subset FFN calls need a run mask and otherwise validate as the calls without one."""
    m = _lib()
    L = m.lib()
    st = _store(m)
    dec = lambda x=FAKE, T=1, mask=FAKE, ws_bytes=1 << 20: L.moe_ffn_fp4_decode_subset(
        x, T, 2, 8, ctypes.byref(st), None, FAKE, FAKE, mask, FAKE, FAKE, ws_bytes, None)
    pre = lambda x=FAKE, T=4, mask=FAKE, act=0, ws_bytes=1 << 30: L.moe_ffn_fp4_prefill_subset(
        x, T, 2, 8, ctypes.byref(st), None, FAKE, FAKE, mask, act, FAKE, FAKE, ws_bytes, None)
    assert dec(mask=None) == m.MOE_ERR_NULL
    assert dec(x=None) == m.MOE_ERR_NULL
    assert dec(ws_bytes=16) == m.MOE_ERR_WORKSPACE
    assert dec(T=300) == m.MOE_ERR_UNSUPPORTED
    assert dec(T=0, mask=None) == m.MOE_OK
    assert pre(mask=None) == m.MOE_ERR_NULL
    assert pre(x=None) == m.MOE_ERR_NULL
    assert pre(act=7) == m.MOE_ERR_UNSUPPORTED
    assert pre(ws_bytes=0) == m.MOE_ERR_WORKSPACE
    assert pre(T=0, mask=None) == m.MOE_OK


def test_packed_prefill_validation():
    """The operand-order copy of the experts: its size, and the pack and packed
    prefill calls' argument checks (no launch is reached)."""
    m = _lib()
    L = m.lib()
    st = _store(m)
    # hidden 256, inter 128: gate and up 4 row blocks x 1 pair, down 8 row blocks x 1 (half-empty) pair
    assert L.moe_prefill_packed_bytes(8, 256, 128) == 8 * 16 * 4352
    # hidden 5120, inter 2304: 2 x 72 x 20 + 160 x 9 blocks of 4352 bytes per slot
    assert L.moe_prefill_packed_bytes(384, 5120, 2304) == 384 * (2 * 72 * 20 + 160 * 9) * 4352
    assert L.moe_prefill_packed_bytes(8, 320, 128) == 0
    assert L.moe_prefill_packed_bytes(8, 256, 96) == 0
    assert L.moe_prefill_packed_bytes(0, 256, 128) == 0
    need = L.moe_prefill_packed_bytes(8, 256, 128)
    assert L.moe_prefill_pack_weights(None, FAKE, need, None) == m.MOE_ERR_NULL
    assert L.moe_prefill_pack_weights(ctypes.byref(st), None, need, None) == m.MOE_ERR_NULL
    assert L.moe_prefill_pack_weights(ctypes.byref(st), MIS, need, None) == m.MOE_ERR_ALIGN
    assert L.moe_prefill_pack_weights(ctypes.byref(st), FAKE, need - 1, None) == m.MOE_ERR_WORKSPACE
    pre = lambda packed=FAKE, pbytes=need, T=4, x=FAKE, ws_bytes=1 << 30: L.moe_ffn_fp4_prefill_packed(
        x, T, 2, 8, ctypes.byref(st), packed, pbytes, None, FAKE, FAKE, 0, FAKE, FAKE, ws_bytes, None)
    assert pre(packed=None) == m.MOE_ERR_NULL
    assert pre(packed=MIS) == m.MOE_ERR_ALIGN
    assert pre(pbytes=need - 1) == m.MOE_ERR_WORKSPACE
    assert pre(x=None) == m.MOE_ERR_NULL
    assert pre(ws_bytes=0) == m.MOE_ERR_WORKSPACE
    assert pre(T=0, packed=None) == m.MOE_OK


def test_prefill_and_combine_validation():
    m = _lib()
    L = m.lib()
    st = _store(m)
    assert L.moe_ffn_fp4_prefill(FAKE, 4, 2, 8, ctypes.byref(st), None, FAKE, FAKE, 7, FAKE, FAKE, 1 << 30,
                                 None) == m.MOE_ERR_UNSUPPORTED                      # unknown activation format
    assert L.moe_ffn_fp4_prefill(None, 4, 2, 8, ctypes.byref(st), None, FAKE, FAKE, 0, FAKE, FAKE, 1 << 30,
                                 None) == m.MOE_ERR_NULL
    assert L.moe_ffn_fp4_prefill(FAKE, 4, 2, 8, ctypes.byref(st), None, FAKE, FAKE, 0, FAKE, FAKE, 0,
                                 None) == m.MOE_ERR_WORKSPACE
    big = _store(m, hidden=16384, inter=8192)
    # 200,000 tokens at hidden 16384: 2.46 GB of MXFP6 x, past 31-bit offsets
    assert L.moe_ffn_fp4_prefill(FAKE, 200000, 1, 8, ctypes.byref(big), None, FAKE, FAKE, 0, FAKE, FAKE, 1 << 40,
                                 None) == m.MOE_ERR_UNSUPPORTED
    # x is quantised once per routed row: 40,000 tokens x top-8 at hidden 16384 is 3.9 GB
    assert L.moe_ffn_fp4_prefill(FAKE, 40000, 8, 8, ctypes.byref(big), None, FAKE, FAKE, 0, FAKE, FAKE, 1 << 40,
                                 None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(None, FAKE, 1, 2, 256, None, 0, FAKE, None) == m.MOE_ERR_NULL
    assert L.moe_combine(FAKE, FAKE, 1, 2, 250, None, 0, FAKE, None) == m.MOE_ERR_SHAPE
    assert L.moe_combine(FAKE, FAKE, 1, 2, 256, None, 5, FAKE, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(MIS, FAKE, 1, 2, 256, None, 0, FAKE, None) == m.MOE_ERR_ALIGN
    assert L.moe_combine(FAKE, FAKE, 1, 2, 256, MIS, 0, FAKE, None) == m.MOE_ERR_ALIGN
    assert L.moe_rmsnorm_bf16(None, 1, 256, 1e-6, FAKE, None) == m.MOE_ERR_NULL
    assert L.moe_rmsnorm_bf16(FAKE, 1, 250, 1e-6, FAKE, None) == m.MOE_ERR_SHAPE
    assert L.moe_rmsnorm_bf16(FAKE, 1, 256, -1.0, FAKE, None) == m.MOE_ERR_SHAPE


def test_python_binding_refuses_cpu_tensors():
    import torch
    m = _lib()
    with pytest.raises(ValueError):
        m.moe_route(torch.zeros((1, 8)), 2)


def _layer_call(m, logits=FAKE, x=FAKE, T=1, E=8, k=2, e2s=None, store=None, res=None, od=0, out=FAKE,
                ids=FAKE, tw=FAKE, ws=FAKE, ws_bytes=1 << 20):
    st = _store(m, hidden=1024, inter=256) if store is None else store
    return m.lib().moe_decode_layer(logits, x, T, E, k, e2s, ctypes.byref(st), res, od, out, ids, tw, ws,
                                    ws_bytes, None)


def _norm_layer_call(m, logits=FAKE, x=FAKE, eps=1e-6, T=1, E=8, k=2, od=0, out=FAKE, ws=FAKE, ws_bytes=1 << 20):
    st = _store(m, hidden=1024, inter=256)
    return m.lib().moe_decode_layer_rmsnorm(logits, x, eps, T, E, k, None, ctypes.byref(st), od, out, FAKE, FAKE, ws,
                                            ws_bytes, None)


def test_decode_layer_rmsnorm_validation():
    m = _lib()
    # the layer's own workspace, then T x hidden bf16 for the normalised rows
    assert m.decode_layer_rmsnorm_workspace_bytes(1, 8, 384, 5120, 2304) == 512 + 8 * 2304 * 4 + 5120 * 2
    lb = m.decode_layer_workspace_bytes(16, 8, 384, 5120, 2304)
    assert m.decode_layer_rmsnorm_workspace_bytes(16, 8, 384, 5120, 2304) == (lb + 255) // 256 * 256 + 16 * 5120 * 2
    assert m.decode_layer_rmsnorm_workspace_bytes(0, 8, 384, 5120, 2304) == 0
    assert _norm_layer_call(m, eps=-1.0) == m.MOE_ERR_SHAPE
    assert _norm_layer_call(m, eps=float("nan")) == m.MOE_ERR_SHAPE
    assert _norm_layer_call(m, x=None) == m.MOE_ERR_NULL
    assert _norm_layer_call(m, x=MIS) == m.MOE_ERR_ALIGN
    need = m.decode_layer_rmsnorm_workspace_bytes(1, 2, 8, 1024, 256)
    assert _norm_layer_call(m, ws_bytes=need - 1) == m.MOE_ERR_WORKSPACE
    assert _norm_layer_call(m, T=0, logits=None, x=None, out=None, ws=None) == m.MOE_OK


def test_decode_layer_validation():
    m = _lib()
    # one token at a fused shape: the routing record plus h in [k][inter] fp32
    assert m.decode_layer_workspace_bytes(1, 8, 384, 5120, 2304) == 512 + 8 * 2304 * 4
    assert m.decode_layer_workspace_bytes(1, 2, 8, 1024, 256) == 512 + 2 * 256 * 4
    # other shapes: offsets, the two pair maps, the permute and h workspaces and y_pair
    assert m.decode_layer_workspace_bytes(16, 8, 384, 5120, 2304) >= 16 * 8 * (5120 + 2304) * 4
    assert m.decode_layer_workspace_bytes(1, 2, 8, 256, 128) >= 2 * (256 + 128) * 4
    assert m.decode_layer_workspace_bytes(0, 2, 8, 256, 128) == 0
    assert _layer_call(m, logits=None) == m.MOE_ERR_NULL
    assert _layer_call(m, out=None) == m.MOE_ERR_NULL
    assert _layer_call(m, ids=None) == m.MOE_ERR_NULL
    assert _layer_call(m, k=9, E=8) == m.MOE_ERR_SHAPE
    assert _layer_call(m, k=0) == m.MOE_ERR_SHAPE
    assert _layer_call(m, E=2000) == m.MOE_ERR_SHAPE
    assert _layer_call(m, store=_store(m, hidden=1000, inter=256)) == m.MOE_ERR_SHAPE
    assert _layer_call(m, store=_store(m, num_slots=4, hidden=1024, inter=256)) == m.MOE_ERR_SHAPE
    assert _layer_call(m, T=300) == m.MOE_ERR_UNSUPPORTED
    assert _layer_call(m, od=5) == m.MOE_ERR_UNSUPPORTED
    assert _layer_call(m, x=MIS) == m.MOE_ERR_ALIGN
    assert _layer_call(m, res=MIS) == m.MOE_ERR_ALIGN
    assert _layer_call(m, ws=None) == m.MOE_ERR_WORKSPACE
    assert _layer_call(m, ws_bytes=512) == m.MOE_ERR_WORKSPACE
    assert _layer_call(m, ws=FAKE + 16) == m.MOE_ERR_ALIGN
    assert _layer_call(m, T=0, logits=None, x=None, out=None, ids=None, tw=None, ws=None) == m.MOE_OK


def test_router_gate_validation():
    """The gate projection calls check shapes, pointers and alignment before any launch."""
    m = _lib()
    L = m.lib()
    lg = lambda x=FAKE, T=4, H=256, w=FAKE, E=8, out=FAKE: L.moe_router_logits(x, T, H, w, E, None, out, None)
    assert lg(x=None) == m.MOE_ERR_NULL
    assert lg(w=None) == m.MOE_ERR_NULL
    assert lg(out=None) == m.MOE_ERR_NULL
    assert lg(H=200) == m.MOE_ERR_SHAPE
    assert lg(H=32768) == m.MOE_ERR_SHAPE
    assert lg(E=0) == m.MOE_ERR_SHAPE
    assert lg(E=2000) == m.MOE_ERR_SHAPE
    assert lg(T=-1) == m.MOE_ERR_SHAPE
    assert lg(x=MIS) == m.MOE_ERR_ALIGN
    assert lg(w=MIS) == m.MOE_ERR_ALIGN
    assert lg(T=1 << 20, H=1024) == m.MOE_ERR_UNSUPPORTED   # x past 31-bit buffer offsets
    assert lg(T=0, x=None) == m.MOE_OK
    rx = lambda T=4, k=2, E=8, ids=FAKE, w=FAKE, out=FAKE: L.moe_route_x(
        FAKE, T, 256, FAKE, E, None, k, None, out, ids, w, None)
    assert rx(k=0) == m.MOE_ERR_SHAPE
    assert rx(k=9) == m.MOE_ERR_SHAPE
    assert rx(k=17, E=64) == m.MOE_ERR_SHAPE
    assert rx(ids=None) == m.MOE_ERR_NULL
    assert rx(w=None) == m.MOE_ERR_NULL
    assert rx(out=None) == m.MOE_ERR_NULL
    assert rx(T=0, ids=None) == m.MOE_OK


def test_cb3_decode_validation():
    """The cb3 decode FFN checks its store, shapes, alignment and workspace before any launch."""
    m = _lib()
    L = m.lib()

    def st(**kw):
        f = dict(num_slots=8, hidden=256, inter=128, q_gate=FAKE, q_up=FAKE, q_down=FAKE,
                 cb_gate=FAKE, cb_up=FAKE, cb_down=FAKE)
        f.update(kw)
        return m.CCb3Experts(f["num_slots"], f["hidden"], f["inter"], f["q_gate"], f["q_up"], f["q_down"],
                                 f["cb_gate"], f["cb_up"], f["cb_down"])

    def call(store=None, x=FAKE, T=1, k=2, E=8, ws=FAKE, ws_bytes=1 << 20):
        s = st() if store is None else store
        return L.moe_ffn_cb3_decode(x, T, k, E, ctypes.byref(s), None, FAKE, FAKE, FAKE, ws, ws_bytes, None)

    assert L.moe_ffn_cb3_decode(FAKE, 1, 2, 8, None, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == m.MOE_ERR_NULL
    assert call(store=st(cb_up=None)) == m.MOE_ERR_NULL
    assert call(x=None) == m.MOE_ERR_NULL
    assert call(store=st(hidden=200)) == m.MOE_ERR_SHAPE
    assert call(store=st(inter=100)) == m.MOE_ERR_SHAPE
    assert call(store=st(hidden=8192)) == m.MOE_ERR_UNSUPPORTED
    assert call(store=st(inter=8192)) == m.MOE_ERR_UNSUPPORTED
    assert call(store=st(q_down=FAKE + 2)) == m.MOE_ERR_ALIGN
    assert call(store=st(cb_gate=FAKE + 8)) == m.MOE_ERR_ALIGN
    assert call(store=st(num_slots=4)) == m.MOE_ERR_SHAPE
    assert call(x=MIS) == m.MOE_ERR_ALIGN
    assert call(ws=None) == m.MOE_ERR_WORKSPACE
    assert call(ws_bytes=16) == m.MOE_ERR_WORKSPACE
    assert call(T=300) == m.MOE_ERR_UNSUPPORTED
    assert call(k=9) == m.MOE_ERR_SHAPE
    assert call(T=0, x=None) == m.MOE_OK
    assert L.moe_ffn_cb3_decode_workspace_bytes(1, 8, 2304) == 8 * 2304 * 4


def test_noalloc_layer_validation():
    """moe_decode_layer_noalloc validates as moe_decode_layer and rejects, before
    any HIP call, a call whose workspace would not fit the static scratch."""
    m = _lib()
    L = m.lib()
    big = _store(m, hidden=5120, inter=2304, num_slots=384)
    call = lambda logits=FAKE, x=FAKE, T=1, E=384, k=8, st=big, od=0, out=FAKE: L.moe_decode_layer_noalloc(
        logits, x, T, E, k, None, ctypes.byref(st), None, od, out, FAKE, FAKE, None)
    assert call(logits=None) == m.MOE_ERR_NULL
    assert call(out=MIS) == m.MOE_ERR_ALIGN
    assert call(od=5) == m.MOE_ERR_UNSUPPORTED
    assert call(k=17) == m.MOE_ERR_SHAPE
    assert call(T=257) == m.MOE_ERR_UNSUPPORTED
    assert call(T=0) == m.MOE_OK
    # 256 tokens need 58 MiB, 128 tokens 29 MiB: the scratch holds 32 MiB
    assert m.decode_layer_workspace_bytes(256, 8, 384, 5120, 2304) > m.NOALLOC_SCRATCH_BYTES
    assert m.decode_layer_workspace_bytes(128, 8, 384, 5120, 2304) <= m.NOALLOC_SCRATCH_BYTES
    assert call(T=256) == m.MOE_ERR_WORKSPACE


def test_invariant_layer_validation():
    """moe_decode_layer_invariant validates as moe_decode_layer, with its own
    workspace size (one token: routing record, h planes and y_pair)."""
    m = _lib()
    L = m.lib()
    # routing record, h planes, y_pair
    assert m.decode_layer_invariant_workspace_bytes(1, 8, 384, 5120, 2304) == 256 + 8 * 2304 * 4 + 8 * 5120 * 4
    assert m.decode_layer_invariant_workspace_bytes(16, 8, 384, 5120, 2304) == \
        m.decode_layer_workspace_bytes(16, 8, 384, 5120, 2304)
    assert m.decode_layer_invariant_workspace_bytes(0, 8, 384, 5120, 2304) == 0
    st = _store(m, hidden=1024, inter=256, num_slots=8)
    need = m.decode_layer_invariant_workspace_bytes(1, 2, 8, 1024, 256)

    def call(logits=FAKE, x=FAKE, T=1, E=8, k=2, store=st, od=0, out=FAKE, ids=FAKE, ws=FAKE, ws_bytes=need):
        return L.moe_decode_layer_invariant(logits, x, T, E, k, None, ctypes.byref(store), None, od, out, ids, FAKE,
                                            ws, ws_bytes, None)
    assert call(logits=None) == m.MOE_ERR_NULL
    assert call(ids=None) == m.MOE_ERR_NULL
    assert call(k=9) == m.MOE_ERR_SHAPE
    assert call(T=300) == m.MOE_ERR_UNSUPPORTED
    assert call(od=5) == m.MOE_ERR_UNSUPPORTED
    assert call(x=MIS) == m.MOE_ERR_ALIGN
    assert call(ws=None) == m.MOE_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == m.MOE_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == m.MOE_ERR_ALIGN
    assert call(T=0, logits=None, x=None, out=None, ids=None, ws=None) == m.MOE_OK
