"""Seeded synthetic inputs for the hybrid-attention workloads.

This package is the only code that both the float64 oracle (``oracle/``) and the
HIP path's tests and benchmark use. It holds none of the attention method's
arithmetic: only random draws, the round-to-nearest-even cast of drawn fp32 values
to bfloat16, the planted-structure construction and the workload constants.
"""

from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits,
    bf16_bits_to_f32,
    round_to_bf16,
    top_k_count,
    frame_block,
    tiny_f32_frames,
    wan_layer_inputs,
    planted_inputs,
    ragged_layer_inputs,
    RAGGED_WINDOW_FRAMES,
    LongStream,
)
