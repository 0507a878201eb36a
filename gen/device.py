"""Device-side placement of the synthetic inputs (torch allocations + the
SplitMix64 device filler in gen/fill.hip).  Input generation only."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import splitmix as sm
from .inputs import Config, HostInputs

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_gen.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python fp4_routed_expert_mxfp4_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        L.gen_fill_codes.argtypes = [vp, i64, vp, i32, u32, i32, i32, vp]
        L.gen_fill_scales.argtypes = [vp, i64, vp, i32, u32, i32, i32, i32, vp]
        L.gen_fill_codes.restype = L.gen_fill_scales.restype = ctypes.c_int
        L.gen_stream_read.argtypes = [vp, i64, vp, vp]
        L.gen_stream_read.restype = ctypes.c_int
        L.gen_stream_read_lds.argtypes = [vp, i64, vp, vp]
        L.gen_stream_read_lds.restype = ctypes.c_int
        L.gen_clock_probe.argtypes = [vp, i32, i32, vp]
        L.gen_clock_probe.restype = ctypes.c_int
        L.gen_load_probe.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.gen_load_probe.restype = ctypes.c_int
        _lib = L
    return _lib


def fill_layer(cfg: Config, layer: int, slot_expert: np.ndarray, device="cuda"):
    """Allocate one layer's expert store and fill slot s with expert slot_expert[s].

    Returns the six uint8 tensors (w_gate, s_gate, w_up, s_up, w_down, s_down).
    """
    S, H, I = len(slot_expert), cfg.H, cfg.I
    dev = torch.device(device)
    se = torch.from_numpy(np.ascontiguousarray(slot_expert, dtype=np.int32)).to(dev)
    shapes = {sm.MATRIX_GATE: (I, H), sm.MATRIX_UP: (I, H), sm.MATRIX_DOWN: (H, I)}
    out = []
    stream = torch.cuda.current_stream(dev).cuda_stream
    for m in (sm.MATRIX_GATE, sm.MATRIX_UP, sm.MATRIX_DOWN):
        rows, K = shapes[m]
        codes = torch.empty((S, rows, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((S, rows, K // 32), dtype=torch.uint8, device=dev)
        rc = lib().gen_fill_codes(codes.data_ptr(), rows * K // 2, se.data_ptr(), S, cfg.seed, layer, m, stream)
        if rc:
            raise RuntimeError(f"gen_fill_codes failed ({rc})")
        rc = lib().gen_fill_scales(scales.data_ptr(), rows * K // 32, se.data_ptr(), S, cfg.seed, layer, m,
                                   cfg.emin, stream)
        if rc:
            raise RuntimeError(f"gen_fill_scales failed ({rc})")
        out += [codes, scales]
    torch.cuda.current_stream(dev).synchronize()
    return tuple(out)


def upload(hi: HostInputs, layer: int = 0, device="cuda"):
    """x (bf16), logits of one layer (fp32) and its expert_to_slot table on the device."""
    dev = torch.device(device)
    x = torch.from_numpy(hi.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(hi.logits[layer]).to(dev)
    e2s = torch.from_numpy(hi.expert_to_slot[layer]).to(dev)
    return x, logits, e2s


def fill_cb3_layer(cfg: Config, layer: int, slot_expert: np.ndarray, device="cuda"):
    """One layer's cb3 expert store: index bytes filled on the device from the
    SplitMix code streams of matrices 8 + m, codebooks generated on the host.

    Returns (q_gate, q_up, q_down, cb_gate, cb_up, cb_down).
    """
    from .inputs import CB3_MATRIX_BASE, cb3_codebook
    S, H, I = len(slot_expert), cfg.H, cfg.I
    dev = torch.device(device)
    se = torch.from_numpy(np.ascontiguousarray(slot_expert, dtype=np.int32)).to(dev)
    shapes = {sm.MATRIX_GATE: (I, H), sm.MATRIX_UP: (I, H), sm.MATRIX_DOWN: (H, I)}
    stream = torch.cuda.current_stream(dev).cuda_stream
    qs, cbs = [], []
    for m in (sm.MATRIX_GATE, sm.MATRIX_UP, sm.MATRIX_DOWN):
        rows, K = shapes[m]
        q = torch.empty((S, rows, K * 3 // 8), dtype=torch.uint8, device=dev)
        rc = lib().gen_fill_codes(q.data_ptr(), rows * K * 3 // 8, se.data_ptr(), S, cfg.seed, layer,
                                  CB3_MATRIX_BASE + m, stream)
        if rc:
            raise RuntimeError(f"gen_fill_codes failed ({rc})")
        cb = np.stack([cb3_codebook(cfg, layer, int(e), m) for e in slot_expert])
        qs.append(q)
        cbs.append(torch.from_numpy(cb.view(np.int16)).to(dev))
    torch.cuda.current_stream(dev).synchronize()
    return tuple(qs + cbs)
