"""MI355X (gfx950) grouped expert MLP: routed top-k permutation, grouped gate-up GEMM,
SwiGLU x routing probability, grouped down GEMM and combine, forward and backward, in
BF16 and MXFP8 — hand-written HIP kernels behind the C ABI in include/mge.h.

The Python names mirror the C entry points; they only marshal arguments and allocate
outputs with torch.  The library must be built (``python -m
moe_grouped_expert_amd.build``); without it every call raises.
"""
from ._binding import (  # noqa: F401
    BwdOut, FwdOut, MgeError, RouteOut, check_device_errors, fwd_saved_bytes, grouped_mlp_bwd, grouped_mlp_fwd,
    grouped_mlp_fwd_unfused,
    lib,
    moe_route_permute, moe_router_bwd, mxfp8_quantize, perm_rows, profile_start, profile_stop, tensor_scale,
    unpermute_combine,
)

__version__ = "0.1.0"
