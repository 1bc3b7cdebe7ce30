"""Seeded synthetic frame generator shared by the oracle, the tests and the bench.

This package produces inputs only. It holds none of the StateKV arithmetic
(attention, importance scores, selection, cache updates): it draws Gaussian
query/key/value tokens, rotates queries and keys at their original positions,
plants early "temporal sink" keys and rounds everything to bfloat16.
"""

from .generator import (  # noqa: F401
    WORKLOADS,
    FrameSpec,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    frame,
    frames,
    hidden_states,
    hidden_width,
    projection_weights,
    rope_rotate,
    sink_plan,
    split_projection_weights,
    stacked_frames,
    text_queries,
    workload,
)
