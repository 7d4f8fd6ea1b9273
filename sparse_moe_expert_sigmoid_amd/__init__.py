"""MI355X (gfx950) sigmoid-routed Q4 MoE expert layer.

The compute lives in the HIP library ``libmoe_q4.so`` (C ABI declared in
``include/moe_q4.h``).  This package is a thin ctypes binding with the same
entry-point names; torch is used only for device buffers and streams.  The
library is loaded on first use and importing fails loudly if it has not
been built (``python -m sparse_moe_expert_sigmoid_amd.build``): there is no
CPU fallback.
"""
from .abi import (  # noqa: F401
    MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EUNSUPPORTED, MOE_ENOSPACE, MOE_EHIP,
    MOE_FLAG_DEFAULT, MOE_FLAG_FORCE_GROUPED, MOE_FLAG_FORCE_GEMV, MOE_FLAG_ID_ORDER,
    MOE_FLAG_NO_BANDING, MOE_GEMV_MAX_T, MoeError, Dims, lib, lib_path,
    moe_supports, moe_path, moe_routing_bytes, moe_routing_layout_of, moe_scratch_bytes,
    moe_route, moe_build_descriptors, moe_q4_forward, moe_q4_forward_residual, moe_layer_forward, moe_strerror,
    EXPORTED_SYMBOLS,
    moe_decode_ctx_workspace_bytes, moe_decode_ctx_create, moe_decode_ctx_run, moe_decode_ctx_destroy,
    moe_rmsnorm_bf16, moe_q4_pack, moe_layer_forward_noalloc, MOE_NOALLOC_MAX_BYTES,
    moe_q4_to_mxfp4, moe_q4_to_mxfp8, moe_rows_to_fp8, moe_w4a8_scratch_bytes, moe_w8a8_scratch_bytes,
    moe_w4a8_forward, moe_w8a8_forward,
)
