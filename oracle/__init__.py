"""CPU oracle of the batched Muon step (test infrastructure only).

Imported by the tests, the smoke check and the CPU-baseline leg of bench.py.
The HIP library and its Python binding never import it.
"""
from .muon_oracle import (  # noqa: F401
    CUBIC, DEFAULT_EPS, QUINTIC, apply_update, frobenius_norm, is_tall, momentum,
    muon_step, nesterov_direction, newton_schulz, normalize, update_scale,
)
from .adamw_oracle import adamw_step  # noqa: F401,E402
