"""Float64 CPU oracle of the optimizer update applied to the expert weights.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the bench's CPU-baseline leg may use it.

What the pages fix and what is read into them
---------------------------------------------
"Support combined expert and data parallelism in TrainerRank" (Acceptance)
asks for a canary that completes forward, backward *and optimizer update*;
"Support pipeline parallelism in TrainerRank without exposing stage
scheduling to callers" (Acceptance) asks that parameter updates match a
matched reference within stated tolerances. Neither page names the
optimizer. The reading taken here is AdamW, Adam with decoupled weight
decay (Loshchilov and Hutter, "Decoupled Weight Decay Regularization"), in
the form PyTorch's ``torch.optim.AdamW`` uses by default (no amsgrad, no
maximize), applied element by element to fp32 master weights:

  g      = grad_scale * grad
  m      = beta1 * m + (1 - beta1) * g
  v      = beta2 * v + (1 - beta2) * g^2
  m_hat  = m / (1 - beta1^t)          (bias corrections, t = 1, 2, ...)
  v_hat  = v / (1 - beta2^t)
  theta  = theta - lr * weight_decay * theta - lr * m_hat / (sqrt(v_hat) + eps)

The decay term uses the weights from before this step, and eps is added
after the square root of the bias-corrected second moment. ``grad_scale``
lets the caller turn the plain gradient sums the layer accumulates into
means (for example 1 / number of microbatches).
"""
from __future__ import annotations

import numpy as np

__all__ = ["adamw_step"]


def adamw_step(theta, grad, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
               grad_scale=1.0):
    """One AdamW step at step number t (1-based) on float64 copies.

    Returns (theta_new, m_new, v_new); the inputs are not modified."""
    if t < 1:
        raise ValueError("the step number t starts at 1")
    theta = np.asarray(theta, dtype=np.float64)
    g = grad_scale * np.asarray(grad, dtype=np.float64)
    m_new = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** t)
    v_hat = v_new / (1.0 - beta2 ** t)
    theta_new = theta - lr * weight_decay * theta - lr * m_hat / (np.sqrt(v_hat) + eps)
    return theta_new, m_new, v_new
