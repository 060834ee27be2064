"""fp64 CPU oracle of the verify / accept / commit step (test infrastructure; see oracle/verify.py).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
"""
from .verify import (  # noqa: F401
    ST_BAD_ACCEPT, ST_BAD_OFFSETS, ST_BAD_Q, ST_BAD_PARENT, ST_BAD_TOKEN, ST_BAD_UNIFORM, ST_NEAR_ALPHA,
    ST_NEAR_CDF, ST_NONFINITE, ST_ZERO_Q, ST_ZERO_RESIDUAL, argmax_lowest, commit_indices, decode_row,
    draw, sanitize_uniform, softmax_T, sparse_q, verify_chain, verify_tree,
)
from . import plan  # noqa: F401,E402  (DSpark verify-length planner and cap_trim)
from . import kv  # noqa: F401,E402  (KV data move of the commit)
from . import tree_build  # noqa: F401,E402  (EAGLE-2 draft-tree construction)
