"""CPU oracle (float64, numpy) of the StateKV streaming video-prefill step.

Test infrastructure only: the test suite, the build entry point's smoke check
and the benchmark's CPU-baseline leg may import it; the GPU library never does.
"""

from .statekv_oracle import (  # noqa: F401
    FrameResult,
    StateKVOracle,
    attention_mass_diagnostics,
    decode_attention,
    decode_bf16,
    frame_attention,
    frame_front_end,
    full_causal_attention,
    importance_scores,
    layer_scores,
    project_frame,
    rope_at_positions,
    round_to_bf16,
    select_most_recent,
    select_top_b,
)
