"""MI355X-native DeepSeekMoE layer (forward and backward): gfx950 HIP kernels behind a C ABI.

The library (libmoe.so, built by ``python -m mixture_experts_ffn_fp32_amd.build``)
does all of the layer's work; this package only marshals arguments to it.
"""
from .moe import (MoEError, STAGE_NAMES, backward_workspace_size, balance_stats, combine,  # noqa: F401
                  dispatch, expert_ffn, layer_backward, layer_forward, layer_forward_static,
                  load_library, route,
                  timing_enable, timing_read, workspace_size)
