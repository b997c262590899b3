"""Float64 CPU oracle for causal kernelized linear attention.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg use it. It imports nothing from the GPU library,
and the GPU library never imports it.
"""
from .kla_oracle import (  # noqa: F401
    FACTOR_KINDS,
    SQRT2,
    decode_sre_chain,
    decode_step,
    factor_weights,
    hybrid_prefill,
    near_tie_ok,
    phi,
    phi_dim,
    phi_factors,
    phi_pairs,
    prefill,
    prefill_backward,
    prefill_backward_rows,
    prefill_bruteforce,
    prefill_bruteforce_rows,
    prefill_chunked,
    prefill_factors_bruteforce,
    prefill_factors_recurrent,
    prefill_recurrent,
    select_topk,
    sre,
    sre_bruteforce,
)
