"""Plain fp64 CPU oracle for the AdamW step of the 1-D parameters.

TEST INFRASTRUCTURE ONLY, like muon_ref: only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it, and it imports nothing
from the product path.

The pages keep the 2-D parameters (which take the Muon update) and the 1-D
ones in separate buffers (the review of "Support Muon sharding optimizer comm
overlap", PaddlePaddle/Paddle pull request 79428, speaks of the 2-D and 1-D
communication buffers of the Muon sharding optimizer), and item 6 of the
HyperParallel FSDP Muon optimizer RFC asks for weight decay in the standard
AdamW style.  The 1-D parameters
are read here as taking AdamW itself: Adam moments with bias correction and
weight decay decoupled from the gradient (Loshchilov and Hutter, "Decoupled
Weight Decay Regularization"), in the form where the decay multiplies the
parameter before the Adam step is subtracted:

    p <- p * (1 - lr * wd)
    m <- b1 * m + (1 - b1) * g
    v <- b2 * v + (1 - b2) * g^2
    p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

t counts steps from 1.  Every operation is one fp64 NumPy expression.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def adamw_step(p, g, m, v, lr: float, b1: float, b2: float, eps: float, wd: float,
               t: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One AdamW step on one tensor; returns (p, m, v) as new fp64 arrays."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    p = p * (1.0 - lr * wd)
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
