"""Plain float64 CPU oracle of the AdamW step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  The HIP library never links, calls
or reads anything here, and nothing here comes from the HIP path.

AdamW trains the parameters Muon does not cover: about 0.5% of the model
("Domyn is training a 1T-parameter MoE on Europe's Jupiter supercomputer, and
published the recipe", §The model and the machine, optimizer row).  The pages
do not spell AdamW out.  The reading taken is Adam with decoupled weight decay
(Loshchilov and Hutter), in the form PyTorch's AdamW takes.  For the step
numbered t >= 1:

  1. p <- p * (1 - lr * wd)                      (decoupled decay)
  2. m <- beta1 * m + (1 - beta1) * g            (first moment)
  3. v <- beta2 * v + (1 - beta2) * g^2          (second moment)
  4. m_hat = m / (1 - beta1^t),  v_hat = v / (1 - beta2^t)
  5. p <- p - lr * m_hat / (sqrt(v_hat) + eps)

Each step is written out in that order, in float64 numpy, elementwise.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def adamw_step(p, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, step: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One AdamW step on one tensor.  Returns (p', m', v')."""
    if step < 1:
        raise ValueError("step numbers start at 1")
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v

