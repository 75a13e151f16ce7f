"""Plain CPU oracle of the AdaLN DiT block (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product library never does.
"""
from .dit_oracle import (  # noqa: F401
    LN_EPS, MOD_CHUNKS, adaln_modulation, attention, block_forward, dequantize_int8, dequantize_int8_groups,
    gelu_tanh, layer_norm, linear, linear_w8a8, modulate, quantize_int8, quantize_int8_groups, rope_3d,
    rope_axis_dims, rope_positions, softmax_rows, stack_forward, token_merge, token_unmerge,
)
