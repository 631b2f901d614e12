"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .loglinear_oracle import (  # noqa: F401
    backward,
    backward_mva,
    decode_step,
    decode_step_mva,
    fenwick_buckets,
    forward,
    forward_mva,
    forward_rows,
    heads_of_qk,
    level_matrix,
    level_of,
    level_rows,
    lssb,
    mask_rows,
    recurrent_forward,
    states_at,
)
