"""fp64 CPU oracle for the Muon / Newton-Schulz hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.  Every function
cites the passage of the pages it follows; see muon_oracle.py.
"""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import (CUBIC, DEFAULT_EPS, widen_bf16, widen_f32, momentum,  # noqa: F401
                          update_direction, frobenius_normalize, step_coefficients,
                          ns_iterate, newton_schulz, ns_batched, muon_step,
                          orthogonality_error, singular_values, rel_frobenius, factored_ns,
                          spectral_cap_update, power_step, muon_step_capped, adamw_step,
                          momentum_recurrence, ssm_momentum,
                          WEYL_STEP, LANCZOS_BREAKDOWN, lanczos_start, lanczos_extremes, spectral_diagnostics)
