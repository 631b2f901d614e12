"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .loglinear_oracle import (  # noqa: F401
    backward,
    decode_step,
    fenwick_buckets,
    forward,
    forward_rows,
    level_matrix,
    level_of,
    level_rows,
    lssb,
    mask_rows,
    recurrent_forward,
    states_at,
)
