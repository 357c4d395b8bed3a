"""CPU oracle for decode-time Sevren Sparse Attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library.
"""

from .ssa_oracle import (  # noqa: F401
    SSA_NORM_K,
    SSA_NORM_Q,
    SSA_SELECT_DISJOINT,
    decode_full,
    decode_sparse,
    prefill_full,
    relu2_attend,
    relu2_weights,
    rms_normalize,
    select_all,
    select_topk_recent,
    softmax_attend,
    widen,
)
