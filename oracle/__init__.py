"""CPU oracles for the Muon optimizer step and the multi-tensor AdamW step
(test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .muon_oracle import (  # noqa: F401
    DEFAULT_COEFFS, NORM_EPS, bf16_bits, bf16_to_f32, bf16_round, nesterov_momentum,
    frobenius_scale, canonical, ns_iteration, newton_schulz, orthogonalize,
    apply_update, muon_step_matrix, muon_step_tensor,
)
