"""kla — causal kernelized linear attention with the rank-one PSD lift, on
AMD MI355X (gfx950).

The computation lives in libkla.so (hand-written HIP kernels behind the C
ABI of include/kla.h); this package only marshals arguments to it:

  prefill         chunked causal prefill over the float32 state (H, s)
  prefill_quadratic  the same outputs in the quadratic (no state) form
  prefill_quadratic_backward  gradients of the prefill (quadratic form)
  decode_step     one recurrent token, optionally with self-recall scoring
  decode_step_deferred  the same token with deferred folds (the state is
                      written once per decode_pending_period() tokens)
  sre_select      self-recall-error scoring and top-k selection
  hybrid_prefill  sliding window + linear state + sparse cache
  hybrid_decode_step  the same three memories, one token at a time
  hybrid_decode_step_static  that step with the library's static scratch
                      (allocates nothing)

``synth`` builds the seeded synthetic workloads.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    KlaError,
    LIB_PATH,
    decode_flush,
    decode_pending_period,
    decode_pending_slots,
    decode_step,
    decode_step_deferred,
    factor_phi_dim,
    hybrid_decode_flush,
    hybrid_decode_pending_slots,
    hybrid_decode_prime,
    hybrid_decode_state,
    hybrid_decode_static_limit,
    hybrid_decode_step,
    hybrid_decode_step_static,
    hybrid_prefill,
    load_library,
    phi_dim,
    prefill,
    prefill_quadratic,
    prefill_quadratic_backward,
    prefill_uses_matrix_cores,
    profile_enable,
    profile_read,
    sre_select,
)

__all__ = ["prefill", "prefill_quadratic", "prefill_quadratic_backward", "decode_step", "decode_step_deferred",
           "decode_flush", "decode_pending_period", "decode_pending_slots", "sre_select", "hybrid_prefill",
           "hybrid_decode_state", "hybrid_decode_step", "hybrid_decode_step_static",
           "hybrid_decode_static_limit", "hybrid_decode_flush", "hybrid_decode_prime",
           "hybrid_decode_pending_slots", "phi_dim", "factor_phi_dim",
           "load_library",
           "KlaError", "EXPORTS", "LIB_PATH", "profile_enable", "profile_read"]
