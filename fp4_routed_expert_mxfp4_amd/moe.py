"""Python binding of the C ABI in include/moe_fp4.h (ctypes).

Argument marshalling only: every step of the routed MoE FFN runs in the HIP
kernels of libmoe_fp4.so.  torch supplies device memory and the current
stream.  The functions carry the C names; outputs that are not passed in are
allocated with torch on the input's device.  If the library has not been
built, every call raises -- there is no other implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp4.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN = 0, 1, 2, 3
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = 4, 5, 6
MOE_OUT_BF16, MOE_OUT_F32 = 0, 1
MOE_ACT_MXFP6_E2M3 = 0
EXPORTED = ("moe_route", "moe_router_logits", "moe_route_x", "moe_ffn_cb3_decode_workspace_bytes", "moe_ffn_cb3_decode", "moe_permute_workspace_bytes", "moe_permute", "moe_ffn_fp4_decode_workspace_bytes", "moe_ffn_fp4_decode",
            "moe_ffn_fp4_decode_gateup", "moe_ffn_fp4_decode_down", "moe_ffn_fp4_decode_subset",
            "moe_ffn_fp4_decode_invariant",
            "moe_decode_layer_workspace_bytes", "moe_decode_layer", "moe_decode_layer_noalloc", "moe_decode_layer_gateup",
            "moe_decode_layer_invariant_workspace_bytes", "moe_decode_layer_invariant",
            "moe_decode_layer_down", "moe_decode_layer_rmsnorm_workspace_bytes", "moe_decode_layer_rmsnorm",
            "moe_ffn_fp4_prefill_workspace_bytes", "moe_ffn_fp4_prefill", "moe_ffn_fp4_prefill_subset",
            "moe_prefill_packed_bytes", "moe_prefill_pack_weights", "moe_ffn_fp4_prefill_packed", "moe_combine",
            "moe_rmsnorm_bf16", "moe_status_string")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: status {status} ({text})")
        self.status = status


class CExperts(ctypes.Structure):
    _fields_ = [("num_slots", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class CCb3Experts(ctypes.Structure):
    _fields_ = [("num_slots", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("q_gate", ctypes.c_void_p), ("q_up", ctypes.c_void_p), ("q_down", ctypes.c_void_p),
                ("cb_gate", ctypes.c_void_p), ("cb_up", ctypes.c_void_p), ("cb_down", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_fp4.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python fp4_routed_expert_mxfp4_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        _LAYER_ARGS = [vp, vp, i32, i32, i32, vp, ctypes.POINTER(CExperts), vp, ctypes.c_int, vp, vp, vp, vp, sz, vp]
        sig = {
            "moe_route": [vp, i32, i32, i32, vp, vp, vp, vp],
            "moe_router_logits": [vp, i32, i32, vp, i32, vp, vp, vp],
            "moe_route_x": [vp, i32, i32, vp, i32, vp, i32, vp, vp, vp, vp, vp],
            "moe_ffn_cb3_decode_workspace_bytes": [i32, i32, i32],
            "moe_ffn_cb3_decode": [vp, i32, i32, i32, ctypes.POINTER(CCb3Experts), vp, vp, vp, vp, vp, sz, vp],
            "moe_permute_workspace_bytes": [i32, i32, i32],
            "moe_permute": [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp],
            "moe_ffn_fp4_decode_workspace_bytes": [i32, i32, i32],
            "moe_ffn_fp4_decode": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, vp, vp, vp, vp, sz, vp],
            "moe_ffn_fp4_decode_gateup": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, vp, vp, vp, vp, sz, vp],
            "moe_ffn_fp4_decode_down": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, vp, vp, vp, vp, sz, vp],
            "moe_ffn_fp4_decode_subset": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, vp, vp, vp, vp, vp, sz,
                                          vp],
            "moe_ffn_fp4_decode_invariant": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, vp, vp, vp, vp, sz,
                                             vp],
            "moe_decode_layer_workspace_bytes": [i32, i32, i32, i32, i32],
            "moe_decode_layer": _LAYER_ARGS,
            "moe_decode_layer_invariant_workspace_bytes": [i32, i32, i32, i32, i32],
            "moe_decode_layer_invariant": _LAYER_ARGS,
            "moe_decode_layer_noalloc": [vp, vp, i32, i32, i32, vp, ctypes.POINTER(CExperts), vp, ctypes.c_int, vp,
                                         vp, vp, vp],
            "moe_decode_layer_gateup": _LAYER_ARGS,
            "moe_decode_layer_down": _LAYER_ARGS,
            "moe_decode_layer_rmsnorm_workspace_bytes": [i32, i32, i32, i32, i32],
            "moe_decode_layer_rmsnorm": [vp, vp, ctypes.c_float, i32, i32, i32, vp, ctypes.POINTER(CExperts),
                                         ctypes.c_int, vp, vp, vp, vp, sz, vp],
            "moe_ffn_fp4_prefill_workspace_bytes": [i32, i32, i32, i32],
            "moe_ffn_fp4_prefill": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, vp, vp, ctypes.c_int,
                                    vp, vp, sz, vp],
            "moe_ffn_fp4_prefill_subset": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, vp, vp, vp,
                                           ctypes.c_int, vp, vp, sz, vp],
            "moe_prefill_packed_bytes": [i32, i32, i32],
            "moe_prefill_pack_weights": [ctypes.POINTER(CExperts), vp, sz, vp],
            "moe_ffn_fp4_prefill_packed": [vp, i32, i32, i32, ctypes.POINTER(CExperts), vp, sz, vp, vp, vp,
                                           ctypes.c_int, vp, vp, sz, vp],
            "moe_combine": [vp, vp, i32, i32, i32, vp, ctypes.c_int, vp, vp],
            "moe_rmsnorm_bf16": [vp, i32, i32, f32, vp, vp],
            "moe_status_string": [ctypes.c_int],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_permute_workspace_bytes.restype = sz
        L.moe_ffn_cb3_decode_workspace_bytes.restype = sz
        L.moe_ffn_fp4_decode_workspace_bytes.restype = sz
        L.moe_ffn_fp4_prefill_workspace_bytes.restype = sz
        L.moe_prefill_packed_bytes.restype = sz
        L.moe_decode_layer_workspace_bytes.restype = sz
        L.moe_decode_layer_invariant_workspace_bytes.restype = sz
        L.moe_decode_layer_rmsnorm_workspace_bytes.restype = sz
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status, status_string(status))


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device):
    return torch.cuda.current_stream(dev).cuda_stream


def _want(t: torch.Tensor, dtypes, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


@dataclass
class ExpertStore:
    """One layer's experts in the checkpoint layout, as device tensors (uint8).

    w_gate, w_up [S][I][H/2]; s_gate, s_up [S][I][H/32];
    w_down [S][H][I/2]; s_down [S][H][I/32].
    """
    w_gate: torch.Tensor
    s_gate: torch.Tensor
    w_up: torch.Tensor
    s_up: torch.Tensor
    w_down: torch.Tensor
    s_down: torch.Tensor

    @property
    def num_slots(self) -> int:
        return self.w_gate.shape[0]

    @property
    def inter(self) -> int:
        return self.w_gate.shape[1]

    @property
    def hidden(self) -> int:
        return self.w_down.shape[1]

    def cstruct(self) -> CExperts:
        for n in ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"):
            _want(getattr(self, n), (torch.uint8,), n)
        return CExperts(self.num_slots, self.hidden, self.inter,
                        _ptr(self.w_gate), _ptr(self.s_gate), _ptr(self.w_up), _ptr(self.s_up),
                        _ptr(self.w_down), _ptr(self.s_down))


def moe_route(logits: torch.Tensor, k: int, expert_to_slot: torch.Tensor | None = None,
              topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None):
    _want(logits, (torch.float32,), "logits")
    T, E = logits.shape
    dev = logits.device
    if expert_to_slot is not None:
        _want(expert_to_slot, (torch.int32,), "expert_to_slot")
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _want(topk_ids, (torch.int32,), "topk_ids")
    _want(topk_w, (torch.float32,), "topk_w")
    _check("moe_route", lib().moe_route(_ptr(logits), T, E, k, _ptr(expert_to_slot), _ptr(topk_ids),
                                        _ptr(topk_w), _stream(dev)))
    return topk_ids, topk_w


def _router_gate_args(x, w_router, bias, logits):
    _want(x, (torch.bfloat16, torch.int16, torch.uint16), "x")
    _want(w_router, (torch.bfloat16, torch.int16, torch.uint16), "w_router")
    T, H = x.shape
    E, H2 = w_router.shape
    if H2 != H:
        raise ValueError("x [T][H] and w_router [E][H] must share H")
    if bias is not None:
        _want(bias, (torch.float32,), "bias")
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _want(logits, (torch.float32,), "logits")
    return T, H, E, logits


def moe_router_logits(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor | None = None,
                      logits: torch.Tensor | None = None) -> torch.Tensor:
    """logits = x . w_router^T (+ bias): x [T][H], w_router [E][H] bf16 bits; fp32 [T][E]."""
    T, H, E, logits = _router_gate_args(x, w_router, bias, logits)
    _check("moe_router_logits", lib().moe_router_logits(_ptr(x), T, H, _ptr(w_router), E, _ptr(bias),
                                                        _ptr(logits), _stream(x.device)))
    return logits


def moe_route_x(x: torch.Tensor, w_router: torch.Tensor, k: int, bias: torch.Tensor | None = None,
                expert_to_slot: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None):
    """Gate projection and top-k routing in one call; returns (logits, topk_ids, topk_w)."""
    T, H, E, logits = _router_gate_args(x, w_router, bias, logits)
    dev = x.device
    if expert_to_slot is not None:
        _want(expert_to_slot, (torch.int32,), "expert_to_slot")
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _want(topk_ids, (torch.int32,), "topk_ids")
    _want(topk_w, (torch.float32,), "topk_w")
    _check("moe_route_x", lib().moe_route_x(_ptr(x), T, H, _ptr(w_router), E, _ptr(bias), k,
                                            _ptr(expert_to_slot), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                            _stream(dev)))
    return logits, topk_ids, topk_w


def permute_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_permute_workspace_bytes(T, k, E))


def moe_permute(topk_ids: torch.Tensor, E: int, expert_offsets: torch.Tensor | None = None,
                sorted_pair: torch.Tensor | None = None, pair_to_row: torch.Tensor | None = None,
                ws: torch.Tensor | None = None):
    _want(topk_ids, (torch.int32,), "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    if expert_offsets is None:
        expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if sorted_pair is None:
        sorted_pair = torch.empty(T * k, dtype=torch.int32, device=dev)
    if pair_to_row is None:
        pair_to_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    for n, t in (("expert_offsets", expert_offsets), ("sorted_pair", sorted_pair), ("pair_to_row", pair_to_row)):
        _want(t, (torch.int32,), n)
    need = permute_workspace_bytes(T, k, E)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if ws is not None:
        _want(ws, (torch.uint8,), "ws")
    _check("moe_permute", lib().moe_permute(_ptr(topk_ids), T, k, E, _ptr(expert_offsets), _ptr(sorted_pair),
                                            _ptr(pair_to_row), _ptr(ws), 0 if ws is None else ws.numel(),
                                            _stream(dev)))
    return expert_offsets, sorted_pair, pair_to_row


def decode_workspace_bytes(T: int, k: int, inter: int) -> int:
    return int(lib().moe_ffn_fp4_decode_workspace_bytes(T, k, inter))


def prefill_workspace_bytes(T: int, k: int, hidden: int, inter: int) -> int:
    return int(lib().moe_ffn_fp4_prefill_workspace_bytes(T, k, hidden, inter))


def _ffn_args(x, k, store, expert_to_slot, expert_offsets, sorted_pair, y_pair):
    _want(x, _BF16, "x")
    _want(expert_offsets, (torch.int32,), "expert_offsets")
    _want(sorted_pair, (torch.int32,), "sorted_pair")
    if expert_to_slot is not None:
        _want(expert_to_slot, (torch.int32,), "expert_to_slot")
    T, H = x.shape
    if y_pair is None:
        y_pair = torch.empty((T * k, H), dtype=torch.float32, device=x.device)
    _want(y_pair, (torch.float32,), "y_pair")
    return T, y_pair


def _decode_call(name, x, k, E, store, expert_to_slot, expert_offsets, sorted_pair, y_pair, ws):
    T, y_pair = _ffn_args(x, k, store, expert_to_slot, expert_offsets, sorted_pair, y_pair)
    need = decode_workspace_bytes(T, k, store.inter)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    _check(name, getattr(lib(), name)(
        _ptr(x), T, k, E, ctypes.byref(cs), _ptr(expert_to_slot), _ptr(expert_offsets), _ptr(sorted_pair),
        _ptr(y_pair), _ptr(ws), ws.numel(), _stream(x.device)))
    return y_pair


@dataclass
class Cb3Store:
    """One layer's experts in the 3-bit per-row codebook format, as device tensors.

    q_gate, q_up uint8 [S][I][3H/8]; q_down uint8 [S][H][3I/8];
    cb_gate, cb_up [S][I][8], cb_down [S][H][8] bf16 bit patterns (int16/uint16/bfloat16).
    """
    q_gate: torch.Tensor
    q_up: torch.Tensor
    q_down: torch.Tensor
    cb_gate: torch.Tensor
    cb_up: torch.Tensor
    cb_down: torch.Tensor

    @property
    def num_slots(self) -> int:
        return self.q_gate.shape[0]

    @property
    def inter(self) -> int:
        return self.q_gate.shape[1]

    @property
    def hidden(self) -> int:
        return self.q_down.shape[1]

    def cstruct(self) -> CCb3Experts:
        for n in ("q_gate", "q_up", "q_down"):
            _want(getattr(self, n), (torch.uint8,), n)
        for n in ("cb_gate", "cb_up", "cb_down"):
            _want(getattr(self, n), _BF16, n)
        return CCb3Experts(self.num_slots, self.hidden, self.inter, _ptr(self.q_gate), _ptr(self.q_up),
                           _ptr(self.q_down), _ptr(self.cb_gate), _ptr(self.cb_up), _ptr(self.cb_down))


def moe_ffn_cb3_decode(x: torch.Tensor, k: int, E: int, store: Cb3Store,
                       expert_to_slot: torch.Tensor | None, expert_offsets: torch.Tensor,
                       sorted_pair: torch.Tensor, y_pair: torch.Tensor | None = None,
                       ws: torch.Tensor | None = None) -> torch.Tensor:
    """Decode expert FFN over cb3 experts; y_pair fp32 [T*k][H] in (token, slot) order."""
    T, y_pair = _ffn_args(x, k, store, expert_to_slot, expert_offsets, sorted_pair, y_pair)
    need = int(lib().moe_ffn_cb3_decode_workspace_bytes(T, k, store.inter))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    _check("moe_ffn_cb3_decode", lib().moe_ffn_cb3_decode(
        _ptr(x), T, k, E, ctypes.byref(cs), _ptr(expert_to_slot), _ptr(expert_offsets), _ptr(sorted_pair),
        _ptr(y_pair), _ptr(ws), ws.numel(), _stream(x.device)))
    return y_pair


def moe_ffn_fp4_decode(x: torch.Tensor, k: int, E: int, store: ExpertStore,
                       expert_to_slot: torch.Tensor | None, expert_offsets: torch.Tensor,
                       sorted_pair: torch.Tensor, y_pair: torch.Tensor | None = None,
                       ws: torch.Tensor | None = None) -> torch.Tensor:
    return _decode_call("moe_ffn_fp4_decode", x, k, E, store, expert_to_slot, expert_offsets, sorted_pair,
                        y_pair, ws)


def moe_ffn_fp4_decode_invariant(x: torch.Tensor, k: int, E: int, store: ExpertStore,
                                 expert_to_slot: torch.Tensor | None, expert_offsets: torch.Tensor,
                                 sorted_pair: torch.Tensor, y_pair: torch.Tensor | None = None,
                                 ws: torch.Tensor | None = None) -> torch.Tensor:
    """The decode FFN with a token's rows bit-identical at every batch size (one token included)."""
    return _decode_call("moe_ffn_fp4_decode_invariant", x, k, E, store, expert_to_slot, expert_offsets,
                        sorted_pair, y_pair, ws)


def moe_ffn_fp4_decode_subset(x: torch.Tensor, k: int, E: int, store: ExpertStore,
                              expert_to_slot: torch.Tensor | None, expert_offsets: torch.Tensor,
                              sorted_pair: torch.Tensor, run_mask: torch.Tensor, y_pair: torch.Tensor | None = None,
                              ws: torch.Tensor | None = None) -> torch.Tensor:
    """The decode FFN over the experts whose ``run_mask`` byte ([E] uint8) is nonzero; the other
    experts' rows of ``y_pair`` are left as they are."""
    T, y_pair = _ffn_args(x, k, store, expert_to_slot, expert_offsets, sorted_pair, y_pair)
    _want(run_mask, (torch.uint8,), "run_mask")
    need = decode_workspace_bytes(T, k, store.inter)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    _check("moe_ffn_fp4_decode_subset", lib().moe_ffn_fp4_decode_subset(
        _ptr(x), T, k, E, ctypes.byref(cs), _ptr(expert_to_slot), _ptr(expert_offsets), _ptr(sorted_pair),
        _ptr(run_mask), _ptr(y_pair), _ptr(ws), ws.numel(), _stream(x.device)))
    return y_pair


def moe_ffn_fp4_decode_gateup(x, k, E, store, expert_to_slot, expert_offsets, sorted_pair, y_pair=None,
                              ws=None) -> torch.Tensor:
    """First kernel of the decode FFN: writes h into ``ws`` (y_pair untouched)."""
    return _decode_call("moe_ffn_fp4_decode_gateup", x, k, E, store, expert_to_slot, expert_offsets,
                        sorted_pair, y_pair, ws)


def moe_ffn_fp4_decode_down(x, k, E, store, expert_to_slot, expert_offsets, sorted_pair, y_pair=None,
                            ws=None) -> torch.Tensor:
    """Second kernel of the decode FFN: reads h from ``ws``, writes y_pair."""
    return _decode_call("moe_ffn_fp4_decode_down", x, k, E, store, expert_to_slot, expert_offsets,
                        sorted_pair, y_pair, ws)


def decode_layer_workspace_bytes(T: int, k: int, E: int, hidden: int, inter: int) -> int:
    return int(lib().moe_decode_layer_workspace_bytes(T, k, E, hidden, inter))


def moe_decode_layer(logits: torch.Tensor, x: torch.Tensor, k: int, store: ExpertStore,
                     expert_to_slot: torch.Tensor | None = None, residual: torch.Tensor | None = None,
                     out_dtype: int = MOE_OUT_BF16, out: torch.Tensor | None = None,
                     topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None, phase: int = 0):
    """route -> permute -> decode FFN -> combine in one call; returns (out, topk_ids, topk_w).
    phase 1 runs only the routing and gate/up half, phase 2 only the down and combine half."""
    _want(logits, (torch.float32,), "logits")
    _want(x, _BF16, "x")
    T, E = logits.shape
    H = x.shape[1]
    dev = x.device
    if expert_to_slot is not None:
        _want(expert_to_slot, (torch.int32,), "expert_to_slot")
    if residual is not None:
        _want(residual, _BF16, "residual")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_OUT_BF16 else torch.float32, device=dev)
    _want(out, _BF16 if out_dtype == MOE_OUT_BF16 else (torch.float32,), "out")
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _want(topk_ids, (torch.int32,), "topk_ids")
    _want(topk_w, (torch.float32,), "topk_w")
    if ws is None:
        ws = torch.empty(max(decode_layer_workspace_bytes(T, k, E, store.hidden, store.inter), 256),
                         dtype=torch.uint8, device=dev)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    name = ("moe_decode_layer", "moe_decode_layer_gateup", "moe_decode_layer_down")[phase]
    _check(name, getattr(lib(), name)(
        _ptr(logits), _ptr(x), T, E, k, _ptr(expert_to_slot), ctypes.byref(cs), _ptr(residual), out_dtype,
        _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(dev)))
    return out, topk_ids, topk_w


def decode_layer_invariant_workspace_bytes(T: int, k: int, E: int, hidden: int, inter: int) -> int:
    return int(lib().moe_decode_layer_invariant_workspace_bytes(T, k, E, hidden, inter))


def moe_decode_layer_invariant(logits: torch.Tensor, x: torch.Tensor, k: int, store: ExpertStore,
                               expert_to_slot: torch.Tensor | None = None, residual: torch.Tensor | None = None,
                               out_dtype: int = MOE_OUT_BF16, out: torch.Tensor | None = None,
                               topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                               ws: torch.Tensor | None = None):
    """The batch-invariant decode layer in one call; returns (out, topk_ids, topk_w)."""
    _want(logits, (torch.float32,), "logits")
    _want(x, _BF16, "x")
    T, E = logits.shape
    H = x.shape[1]
    dev = x.device
    if expert_to_slot is not None:
        _want(expert_to_slot, (torch.int32,), "expert_to_slot")
    if residual is not None:
        _want(residual, _BF16, "residual")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_OUT_BF16 else torch.float32, device=dev)
    _want(out, _BF16 if out_dtype == MOE_OUT_BF16 else (torch.float32,), "out")
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _want(topk_ids, (torch.int32,), "topk_ids")
    _want(topk_w, (torch.float32,), "topk_w")
    if ws is None:
        ws = torch.empty(max(decode_layer_invariant_workspace_bytes(T, k, E, store.hidden, store.inter), 256),
                         dtype=torch.uint8, device=dev)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    _check("moe_decode_layer_invariant", lib().moe_decode_layer_invariant(
        _ptr(logits), _ptr(x), T, E, k, _ptr(expert_to_slot), ctypes.byref(cs), _ptr(residual), out_dtype,
        _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(dev)))
    return out, topk_ids, topk_w


NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES of the C header


def moe_decode_layer_noalloc(logits: torch.Tensor, x: torch.Tensor, k: int, store: ExpertStore,
                             expert_to_slot: torch.Tensor | None = None, residual: torch.Tensor | None = None,
                             out_dtype: int = MOE_OUT_BF16, out: torch.Tensor | None = None,
                             topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None):
    """moe_decode_layer on the library's static scratch (no workspace argument).
    Returns (out, topk_ids, topk_w); out, topk_ids and topk_w are allocated here
    only when not given."""
    _want(logits, (torch.float32,), "logits")
    _want(x, _BF16, "x")
    T, E = logits.shape
    H = x.shape[1]
    dev = x.device
    if expert_to_slot is not None:
        _want(expert_to_slot, (torch.int32,), "expert_to_slot")
    if residual is not None:
        _want(residual, _BF16, "residual")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_OUT_BF16 else torch.float32, device=dev)
    _want(out, _BF16 if out_dtype == MOE_OUT_BF16 else (torch.float32,), "out")
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _want(topk_ids, (torch.int32,), "topk_ids")
    _want(topk_w, (torch.float32,), "topk_w")
    cs = store.cstruct()
    _check("moe_decode_layer_noalloc", lib().moe_decode_layer_noalloc(
        _ptr(logits), _ptr(x), T, E, k, _ptr(expert_to_slot), ctypes.byref(cs), _ptr(residual), out_dtype,
        _ptr(out), _ptr(topk_ids), _ptr(topk_w), _stream(dev)))
    return out, topk_ids, topk_w


def decode_layer_rmsnorm_workspace_bytes(T: int, k: int, E: int, hidden: int, inter: int) -> int:
    return int(lib().moe_decode_layer_rmsnorm_workspace_bytes(T, k, E, hidden, inter))


def moe_decode_layer_rmsnorm(logits: torch.Tensor, x: torch.Tensor, k: int, store: ExpertStore, eps: float = 1e-6,
                             expert_to_slot: torch.Tensor | None = None, out_dtype: int = MOE_OUT_BF16,
                             out: torch.Tensor | None = None, topk_ids: torch.Tensor | None = None,
                             topk_w: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """One chained decode layer: x is the raw bf16 residual row(s); the layer runs on
    rmsnorm(x) and adds x back.  Returns (out, topk_ids, topk_w)."""
    _want(logits, (torch.float32,), "logits")
    _want(x, _BF16, "x")
    T, E = logits.shape
    H = x.shape[1]
    dev = x.device
    if expert_to_slot is not None:
        _want(expert_to_slot, (torch.int32,), "expert_to_slot")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_OUT_BF16 else torch.float32, device=dev)
    _want(out, _BF16 if out_dtype == MOE_OUT_BF16 else (torch.float32,), "out")
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(decode_layer_rmsnorm_workspace_bytes(T, k, E, store.hidden, store.inter), 256),
                         dtype=torch.uint8, device=dev)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    _check("moe_decode_layer_rmsnorm", lib().moe_decode_layer_rmsnorm(
        _ptr(logits), _ptr(x), float(eps), T, E, k, _ptr(expert_to_slot), ctypes.byref(cs), out_dtype, _ptr(out),
        _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(dev)))
    return out, topk_ids, topk_w


def moe_ffn_fp4_prefill(x: torch.Tensor, k: int, E: int, store: ExpertStore,
                        expert_to_slot: torch.Tensor | None, expert_offsets: torch.Tensor,
                        sorted_pair: torch.Tensor, y_pair: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None, act: int = MOE_ACT_MXFP6_E2M3) -> torch.Tensor:
    T, y_pair = _ffn_args(x, k, store, expert_to_slot, expert_offsets, sorted_pair, y_pair)
    need = prefill_workspace_bytes(T, k, store.hidden, store.inter)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    _check("moe_ffn_fp4_prefill", lib().moe_ffn_fp4_prefill(
        _ptr(x), T, k, E, ctypes.byref(cs), _ptr(expert_to_slot), _ptr(expert_offsets), _ptr(sorted_pair),
        act, _ptr(y_pair), _ptr(ws), ws.numel(), _stream(x.device)))
    return y_pair


def prefill_packed_bytes(num_slots: int, hidden: int, inter: int) -> int:
    """Bytes of the experts' copy in MFMA operand order (0: unsupported shape)."""
    return int(lib().moe_prefill_packed_bytes(num_slots, hidden, inter))


def moe_prefill_pack_weights(store: ExpertStore, packed: torch.Tensor | None = None) -> torch.Tensor:
    """Write the copy of ``store`` that moe_ffn_fp4_prefill_packed's tiled GEMMs read."""
    need = prefill_packed_bytes(store.num_slots, store.hidden, store.inter)
    dev = store.w_gate.device
    if packed is None:
        packed = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _want(packed, (torch.uint8,), "packed")
    cs = store.cstruct()
    _check("moe_prefill_pack_weights", lib().moe_prefill_pack_weights(
        ctypes.byref(cs), _ptr(packed), packed.numel(), _stream(dev)))
    return packed


def moe_ffn_fp4_prefill_packed(x: torch.Tensor, k: int, E: int, store: ExpertStore, packed: torch.Tensor,
                               expert_to_slot: torch.Tensor | None, expert_offsets: torch.Tensor,
                               sorted_pair: torch.Tensor, y_pair: torch.Tensor | None = None,
                               ws: torch.Tensor | None = None, act: int = MOE_ACT_MXFP6_E2M3) -> torch.Tensor:
    """moe_ffn_fp4_prefill with the tiled GEMMs on ``packed`` (moe_prefill_pack_weights of the same store)."""
    T, y_pair = _ffn_args(x, k, store, expert_to_slot, expert_offsets, sorted_pair, y_pair)
    need = prefill_workspace_bytes(T, k, store.hidden, store.inter)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _want(ws, (torch.uint8,), "ws")
    _want(packed, (torch.uint8,), "packed")
    cs = store.cstruct()
    _check("moe_ffn_fp4_prefill_packed", lib().moe_ffn_fp4_prefill_packed(
        _ptr(x), T, k, E, ctypes.byref(cs), _ptr(packed), packed.numel(), _ptr(expert_to_slot),
        _ptr(expert_offsets), _ptr(sorted_pair), act, _ptr(y_pair), _ptr(ws), ws.numel(), _stream(x.device)))
    return y_pair


def moe_ffn_fp4_prefill_subset(x: torch.Tensor, k: int, E: int, store: ExpertStore,
                               expert_to_slot: torch.Tensor | None, expert_offsets: torch.Tensor,
                               sorted_pair: torch.Tensor, run_mask: torch.Tensor,
                               y_pair: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                               act: int = MOE_ACT_MXFP6_E2M3) -> torch.Tensor:
    """The prefill FFN over the experts whose ``run_mask`` byte is nonzero (see the decode form)."""
    T, y_pair = _ffn_args(x, k, store, expert_to_slot, expert_offsets, sorted_pair, y_pair)
    _want(run_mask, (torch.uint8,), "run_mask")
    need = prefill_workspace_bytes(T, k, store.hidden, store.inter)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _want(ws, (torch.uint8,), "ws")
    cs = store.cstruct()
    _check("moe_ffn_fp4_prefill_subset", lib().moe_ffn_fp4_prefill_subset(
        _ptr(x), T, k, E, ctypes.byref(cs), _ptr(expert_to_slot), _ptr(expert_offsets), _ptr(sorted_pair),
        _ptr(run_mask), act, _ptr(y_pair), _ptr(ws), ws.numel(), _stream(x.device)))
    return y_pair


def moe_combine(y_pair: torch.Tensor, topk_w: torch.Tensor, residual: torch.Tensor | None = None,
                out_dtype: int = MOE_OUT_BF16, out: torch.Tensor | None = None) -> torch.Tensor:
    _want(y_pair, (torch.float32,), "y_pair")
    _want(topk_w, (torch.float32,), "topk_w")
    T, k = topk_w.shape
    H = y_pair.shape[1]
    if residual is not None:
        _want(residual, _BF16, "residual")
    if out is None:
        dt = torch.bfloat16 if out_dtype == MOE_OUT_BF16 else torch.float32
        out = torch.empty((T, H), dtype=dt, device=y_pair.device)
    _want(out, _BF16 if out_dtype == MOE_OUT_BF16 else (torch.float32,), "out")
    _check("moe_combine", lib().moe_combine(_ptr(y_pair), _ptr(topk_w), T, k, H, _ptr(residual), out_dtype,
                                            _ptr(out), _stream(y_pair.device)))
    return out


def moe_rmsnorm_bf16(x: torch.Tensor, eps: float = 1e-6, out: torch.Tensor | None = None) -> torch.Tensor:
    _want(x, _BF16, "x")
    T, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    _want(out, _BF16, "out")
    _check("moe_rmsnorm_bf16", lib().moe_rmsnorm_bf16(_ptr(x), T, H, eps, _ptr(out), _stream(x.device)))
    return out
