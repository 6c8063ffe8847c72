"""Float64 CPU oracle of the MoE auxiliary losses and routing metrics.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the bench's CPU-baseline leg may use it.

What the pages fix and what is read into them
---------------------------------------------
"Add MoE expert parallel training runtime" lists MoE metrics among the
training features and MoE losses among the regression coverage (Major
changes), and runs a MoE-losses test module (Validation), without
defining either. The readings taken here are the two standard router
losses and a set of load statistics:

* load-balancing loss (Fedus, Zoph and Shazeer, "Switch Transformers",
  Section 2.2), extended to top-k by counting every routed slot:
      f_e   = counts[e] / (T * k)        fraction of routed rows on expert e
      P_e   = (1/T) sum_t p[t, e]         mean full-softmax probability
      L_bal = E * sum_e f_e * P_e         (= 1 for perfectly even routing)
  f is piecewise constant in the logits, so only P carries gradient:
      dL_bal/dp[t, e] = E * f_e / T.
* router z-loss (Zoph et al., "ST-MoE", Section 3.1):
      L_z = (1/T) sum_t (log sum_e exp(logits[t, e]))^2,
      dL_z/dlogits[t, i] = (2/T) * lse_t * p[t, i].
* the gradient returned is that of alpha * L_bal + beta * L_z with respect
  to the logits; the probabilities' part goes through the softmax Jacobian
  dlogits[t, i] = p_i * (g_i - sum_e p_e g_e).
* metrics, from the counts and the full softmax p of every token:
      imbalance      max_e counts[e] / (T * k / E)
      empty_experts  number of e with counts[e] == 0
      count_cv       standard deviation / mean of counts (population std)
      entropy        (1/T) sum_t -sum_e p[t,e] log p[t,e]   (0 log 0 = 0)
      max_prob       (1/T) sum_t max_e p[t,e]
  followed by f_e and P_e for every expert.

Both losses use the softmax over all E experts whatever the renormalisation
of the routing weights.

An empty microbatch (T = 0) has to run and contribute zero ("Support
combined expert and data parallelism in TrainerRank", Acceptance, the
empty-work case). Its token sums (sum_t lse^2, sum_t p, the counts) are empty
sums, so the reading taken is: both losses 0, every metric 0 except
empty_experts = E, f_e = P_e = 0, and no gradient rows. A caller adding the
losses of several microbatches then adds nothing for the empty one.
"""
from __future__ import annotations

import numpy as np

__all__ = ["aux_losses", "aux_losses_grad", "routing_metrics", "METRIC_NAMES"]

METRIC_NAMES = ("imbalance", "empty_experts", "count_cv", "entropy", "max_prob")


def _softmax_lse(logits):
    z = np.asarray(logits, dtype=np.float64)
    m = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - m)
    s = np.sum(e, axis=1, keepdims=True)
    return e / s, (m + np.log(s))[:, 0]


def aux_losses(logits, counts, k):
    """(L_bal, L_z) of one microbatch (unweighted); (0, 0) when T = 0."""
    if np.asarray(logits).shape[0] == 0:
        return 0.0, 0.0
    p, lse = _softmax_lse(logits)
    T, E = p.shape
    f = np.asarray(counts, dtype=np.float64) / (T * k)
    P = p.mean(axis=0)
    return E * float(np.sum(f * P)), float(np.mean(lse * lse))


def aux_losses_grad(logits, counts, k, alpha, beta):
    """d(alpha L_bal + beta L_z) / dlogits, shape [T, E]."""
    p, lse = _softmax_lse(logits)
    T, E = p.shape
    f = np.asarray(counts, dtype=np.float64) / (T * k)
    g = np.broadcast_to(alpha * E * f / T, p.shape)               # dL/dp from the balance loss
    d_bal = p * (g - np.sum(p * g, axis=1, keepdims=True))        # through the softmax
    d_z = beta * (2.0 / T) * lse[:, None] * p
    return d_bal + d_z


def routing_metrics(logits, counts, k):
    """Array [5 + 2E]: the five scalars of METRIC_NAMES, then f_e, then P_e.
    For T = 0: zeros, except empty_experts = E."""
    T, E = np.asarray(logits).shape
    if T == 0:
        out = np.zeros(5 + 2 * E)
        out[1] = float(E)
        return out
    p, _ = _softmax_lse(logits)
    c = np.asarray(counts, dtype=np.float64)
    mean = T * k / E
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    scalars = [
        float(np.max(c) / mean),
        float(np.sum(c == 0)),
        float(np.sqrt(np.mean((c - mean) ** 2)) / mean),
        float(np.mean(-np.sum(plogp, axis=1))),
        float(np.mean(np.max(p, axis=1))),
    ]
    return np.concatenate([scalars, c / (T * k), p.mean(axis=0)])
