"""Routed MoE FFN over MXFP4 experts on AMD Instinct MI355X (gfx950).

The computation lives in HIP kernels behind the C ABI of include/moe_fp4.h
(libmoe_fp4.so); this package is its Python binding.
"""
from .moe import (  # noqa: F401
    MOE_ACT_MXFP6_E2M3, MOE_OUT_BF16, MOE_OUT_F32, NOALLOC_SCRATCH_BYTES, Cb3Store, ExpertStore, MoeError, decode_workspace_bytes, lib,
    decode_layer_workspace_bytes, decode_layer_rmsnorm_workspace_bytes, decode_layer_invariant_workspace_bytes,
    moe_combine, moe_decode_layer, moe_decode_layer_invariant, moe_decode_layer_noalloc, moe_decode_layer_rmsnorm, moe_ffn_cb3_decode, moe_ffn_fp4_decode, moe_ffn_fp4_decode_down, moe_ffn_fp4_decode_gateup,
    moe_ffn_fp4_decode_invariant, moe_ffn_fp4_decode_subset, moe_ffn_fp4_prefill, moe_ffn_fp4_prefill_packed, moe_ffn_fp4_prefill_subset, moe_permute,
    moe_prefill_pack_weights, moe_rmsnorm_bf16, prefill_packed_bytes,
    moe_route, moe_route_x, moe_router_logits, permute_workspace_bytes, prefill_workspace_bytes, status_string)
