"""CPU oracle for the Sparse GQA forward path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this package.
The GPU product path never imports, calls or links anything here, and nothing here imports the GPU
path: the two share no code.
"""
from .sgqa_oracle import (  # noqa: F401
    num_blocks,
    n_selected_blocks,
    query_positions,
    compress,
    block_scores,
    select_blocks,
    attended_tokens,
    gated_attention,
    forward_rows,
    forward,
    scored_candidates,
    inclusion_rate,
    sequence_rows,
    window_rows,
    e4m3_decode,
    attention_backward,
    attention_lse,
)
