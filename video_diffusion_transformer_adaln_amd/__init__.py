"""MI355X-native forward pass of the AdaLN-modulated DiT block (h3k).

The compute lives in ``libh3k.so`` (HIP kernels for gfx950 behind the C ABI in
``include/h3k.h``); this package holds its ctypes binding and a small
device-memory helper built on torch tensors.
"""
from .binding import (  # noqa: F401
    EXPORTED, H3K_BF16, H3K_EPI_BIAS, H3K_EPI_GATED_RESIDUAL, H3K_EPI_GELU, H3K_ERR_ALIGN, H3K_ERR_DTYPE,
    H3K_ERR_HIP, H3K_ERR_NULL, H3K_ERR_OVERLAP, H3K_ERR_SHAPE, H3K_ERR_UNSUPPORTED, H3K_ERR_WORKSPACE, H3K_F32,
    H3K_INT8, H3K_OK, KERNEL_KINDS, TENSOR_NAMES, DitBlockWeights, DitConfig, DitPlanInfo, DitStats, H3KError,
    Profiler, check, h3k_adaln_modulation, h3k_attention, h3k_dit_block_forward, h3k_dit_plan,
    h3k_dit_stack_forward, h3k_dit_workspace_size, h3k_linear, h3k_ln_modulate, h3k_quantize_weights_int8,
    last_error, lib, make_config, make_weights,
)
