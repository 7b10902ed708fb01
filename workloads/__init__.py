"""Seeded synthetic inputs for the block-diffusion decode round.

This package is shared by the CPU oracle's tests and by the HIP path's tests
and benchmark.  It holds input construction only: counter-keyed random
numbers, bf16 rounding of stored tensors (by torch's own conversion), the
shapes of each workload, and the planting of confidence peaks.  It contains
none of the decode method's arithmetic (no normalisation, routing, expert
FFN, softmax or commit).
"""

from .gen import (  # noqa: F401
    Dims,
    C0,
    C1,
    LMHEAD_C3,
    counter_words,
    counter_uniform,
    counter_normal,
    key_of,
    layer_weights,
    layer_weights_int4,
    int4_matrix,
    router_weights,
    lm_head_weight,
    lm_head_rows,
    lm_head_int4,
    quantize_int4,
    block_hidden,
    zipf_router_bias,
    lmhead_stub_inputs,
    planted_round_inputs,
)
