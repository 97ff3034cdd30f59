"""Float64 CPU oracle (test infrastructure only; see hf_oracle's header)."""
from .hf_oracle import *  # noqa: F401,F403
from .hf_oracle import (  # noqa: F401
    phi, state_init, absorb, block_ranges, block_means, block_scores, select,
    select_from_scores, near_tie_rows, valid_top_k, attend_with_sel, attend,
    stream_step_frames, as_f64, DEFAULT_EPS, linear_read, rope_positions, rope_rotate,
    attend_rope, attend_ragged)
from .hf_oracle_bwd import phi_prime, attend_with_sel_backward, absorb_backward  # noqa: F401
