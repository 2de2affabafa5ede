"""Oracle for the projected Adam step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests and the benchmark call it.  It shares no code with
the GPU library.

What it computes (Memory-Efficient Differentially Private Training with
Gradient Random Projection, English explainer, Methodology, "Projected
Optimizer States": Adam's first and second moments are kept in the projected
r-dimensional space; the step reaches the weight through the projection P
that produced the projected gradient):

  m <- beta1 m + (1 - beta1) h
  v <- beta2 v + (1 - beta2) h^2
  U  = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
  W <- W - lr * U P^T

with h [dout, r] the privatised projected gradient, t the step number
(1 for the first) and P [din, r].  Plain Adam: no weight decay, no AMSGrad.
Everything in float64.
"""
from __future__ import annotations

import numpy as np


def adam_direction(m, v, step: int, beta1: float, beta2: float, eps: float):
    """U = m_hat / (sqrt(v_hat) + eps) with the bias corrections of step t."""
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    return (m / bc1) / (np.sqrt(v / bc2) + eps)


def projected_adam_step(grad, m, v, W, step: int, lr: float, beta1: float, beta2: float,
                        eps: float, P):
    """One step; returns (m, v, W) new, all float64.  P is float64 [din, r]."""
    h = np.asarray(grad, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * h
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * h * h
    U = adam_direction(m, v, step, beta1, beta2, eps)
    W = np.asarray(W, dtype=np.float64) - lr * (U @ np.asarray(P, dtype=np.float64).T)
    return m, v, W
