"""CPU oracle for the dynamic-visual-fixation decode attention path.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  The GPU library
never calls it and shares no code with it.
"""

from .fastocr_oracle import (  # noqa: F401
    kv_head_of,
    attention_probs,
    full_attention,
    sparse_attention,
    image_rows_of,
    image_scores,
    image_mass,
    kept_count,
    select_top,
    choose_focal_layers,
    DecodeOracle,
)
