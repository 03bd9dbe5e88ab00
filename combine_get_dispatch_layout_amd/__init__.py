"""MI355X-native MoE expert-parallel token shuffle: routing layout, slot
assignment, dispatch (optionally FP8 E4M3FN / int8 quantised) and weighted
combine, as hand-written HIP kernels for gfx950 behind a C ABI
(include/ep.h).  This package holds the kernels (csrc/), their build script
and the thin Python binding (ep.py)."""
from .ep import (Config, EpError, Handle, ep_check_error, ep_combine, ep_dispatch,  # noqa: F401
                 ep_get_layout, ep_handle_free, ep_handle_get_view, ep_handle_init,
                 ep_layout_dispatch, ep_quantize_rows, ep_dispatch_topk, ep_dispatch_overlap,
                 ep_combine_overlap,
                 ep_recv_capacity, ep_workspace_size, EP_QUANT_NONE, EP_QUANT_FP8_E4M3,
                 EP_QUANT_INT8, EP_QUANT_MXFP4, EP_SCALE_FP32, EP_SCALE_POW2, EP_SCALE_UE8M0)
