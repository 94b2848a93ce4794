"""MXFP4 MoE expert layer (router, top-k, permutation, MXFP4 gate/up + SwiGLU,
MXFP4 down, gated combine) as hand-written HIP kernels for AMD MI355X (gfx950),
behind the C ABI of include/moe_mxfp4.h.  This package is the thin Python
binding; it raises on import if the HIP library has not been built."""
from .binding import (  # noqa: F401
    LIB_PATH, MOE_EALIGN, MOE_EDEVICE, MOE_EINVAL, MOE_ELAUNCH, MOE_EWORKSPACE, MOE_ESHAPE, MOE_ETIMEOUT, MOE_OK,
    MOE_LAYERS_COOPERATIVE, MOE_LAYERS_ONE_LAUNCH, MOE_LAYERS_PER_LAUNCH, MOE_OPT_COOPERATIVE, MOE_OPT_TRACE, MOE_OPT_WITHHOLD_ARRIVAL, MOE_OPT_WITHHOLD_H,
    MOE_QDTYPE_BF16, MOE_QDTYPE_F32, LayerDims, MoeError, Options, alloc_workspace, dims_of, expert_packed_bytes,
    expert_scale_bytes, forward, forward_layers, forward_noalloc, forward_layers_raw, forward_raw, intermediates, layers_one_launch,
    persistent_grid, quantize, quantize_host, dequantize_host, route, status, strerror,
    workspace_bytes, workspace_init, workspace_layout,
)
