"""CPU oracle for Block Sparse Attention (test infrastructure only; see bsa_oracle)."""
from .bsa_oracle import *  # noqa: F401,F403
from .bsa_oracle import (Problem, ProblemError, check_problem, num_selected,  # noqa: F401
                         segment_cube_tokens, noise_cube_tokens, cond_cube_tokens, block_pool,
                         block_scores, select_row, select_topr, boundary_gap, attn_fwd_row,
                         attn_fwd_rows, sparse_attn_fwd, attn_bwd, delta_rows,
                         transpose_selection, full_block_causal_fwd)
from . import prologue  # noqa: F401
from .prologue import axis_widths, token_positions, rms_norm, rope_3d, qk_prologue  # noqa: F401
