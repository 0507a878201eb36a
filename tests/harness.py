"""Shared helpers of the parity tests: error metrics, device set-up of a
config layer, and running the C-ABI path end to end."""
from __future__ import annotations

import numpy as np
import torch

from gen import device as gd
from gen import inputs as gi

# Tolerance on the MoE output: max|out - ref| / max|ref| over a call.
REL_TOL = 2e-3
# Routing weights: absolute tolerance against the fp64 oracle.
W_TOL = 1e-6
# Prefill against the unquantised (a16) definition, max|out - ref| / max|ref|.
# The prefill arithmetic quantises x and h to MXFP6 (three mantissa bits):
# each element is rounded by at most half its quantum, a relative RMS of about
# 2-3 % on N(0,1)-like blocks, and the two roundings leave the output about
# 4-6 % of max|ref| away from the a16 result (measured 0.038-0.063 over the
# prefill parity shapes).  The bound is a regression guard on that precision:
# losing one mantissa bit in either quantisation roughly doubles the distance.
PREFILL_A16_BOUND = 0.08


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(out - ref)) / (den if den > 0 else 1.0))


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_excess(out_bits: np.ndarray, ref: np.ndarray) -> float:
    """Error of a bf16 store beyond its own rounding: max(0, |out-ref| - half an
    ulp of bf16 at the larger magnitude), relative to max|ref|."""
    out = bf16_to_f64(out_bits)
    ref = np.asarray(ref, np.float64)
    mag = np.maximum(np.abs(out), np.abs(ref))
    e = np.frexp(mag)[1] - 1
    half = np.where(mag > 0, np.ldexp(1.0, np.maximum(e - 8, -134)), 0.0)
    ex = np.maximum(0.0, np.abs(out - ref) - half)
    den = np.max(np.abs(ref))
    return float(np.max(ex) / (den if den > 0 else 1.0))


class GpuLayer:
    """One config layer on the device: filled expert store plus x and logits."""

    def __init__(self, cfg: gi.Config, layer: int = 0, hi: gi.HostInputs | None = None, device="cuda"):
        from fp4_routed_expert_mxfp4_amd import ExpertStore
        self.cfg, self.layer = cfg, layer
        self.hi = hi if hi is not None else gi.host_inputs(cfg)
        self.store = ExpertStore(*gd.fill_layer(cfg, layer, self.hi.resident[layer], device))
        self.x, self.logits, e2s = gd.upload(self.hi, layer, device)
        self.e2s = None if cfg.resident is None else e2s
        self.e2s_np = None if cfg.resident is None else self.hi.expert_to_slot[layer]
        self.weights = gi.HostWeights(cfg, layer)

    def run(self, path: str = "decode", x=None, logits=None, residual=None, out_dtype=None):
        """route -> permute -> FFN (decode, prefill or prefill_packed) -> combine, all on the device."""
        import fp4_routed_expert_mxfp4_amd as m
        cfg = self.cfg
        x = self.x if x is None else x
        logits = self.logits if logits is None else logits
        ids, w = m.moe_route(logits, cfg.k, self.e2s)
        off, sp, p2r = m.moe_permute(ids, cfg.E)
        if path == "prefill_packed":  # the prefill FFN on the experts' operand-order copy
            packed = m.moe_prefill_pack_weights(self.store)
            y = m.moe_ffn_fp4_prefill_packed(x, cfg.k, cfg.E, self.store, packed, self.e2s, off, sp)
        else:
            ffn = m.moe_ffn_fp4_decode if path == "decode" else m.moe_ffn_fp4_prefill
            y = ffn(x, cfg.k, cfg.E, self.store, self.e2s, off, sp)
        out32 = m.moe_combine(y, w, residual, m.MOE_OUT_F32)
        out16 = m.moe_combine(y, w, residual, m.MOE_OUT_BF16)
        torch.cuda.synchronize()
        return dict(ids=ids, w=w, offsets=off, sorted_pair=sp, pair_to_row=p2r, y_pair=y,
                    out32=out32, out16=out16)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
