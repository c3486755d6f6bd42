"""fp64 oracle of one LAMB optimizer step.

Test infrastructure only (see the package docstring).

Source: MegaScale study guide, ch.2 §2.2 (paper §3.1), table of the three
algorithmic changes, LAMB row: a layer-wise adaptive trust ratio (the method
of You et al. 2020) that lets MegaScale grow the batch.  The page gives no
equations, so the steps are those of the published method:

  for every parameter tensor ("layer") separately, at step t >= 1:
    m <- beta1 * m + (1 - beta1) * g
    v <- beta2 * v + (1 - beta2) * g^2
    m_hat = m / (1 - beta1^t),  v_hat = v / (1 - beta2^t)
    u = m_hat / (sqrt(v_hat) + eps) + weight_decay * w
    r = ||w||_2 / ||u||_2, and r = 1 when either norm is zero
    w <- w - lr * r * u

Readings where the page is silent: bias correction on; eps outside the
square root; weight decay added to the update before the norm; the scaling
function of ||w|| is the identity (no clamp); "layer" = one parameter tensor.
"""
from __future__ import annotations

import numpy as np


def lamb_tensor_step(w, g, m, v, step, lr, beta1, beta2, eps, weight_decay):
    """One step for one tensor.  Returns (w_new, m_new, v_new, ratio, u)."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    u = m_hat / (np.sqrt(v_hat) + eps) + weight_decay * w
    w_norm = float(np.sqrt(np.sum(w * w)))
    u_norm = float(np.sqrt(np.sum(u * u)))
    ratio = w_norm / u_norm if (w_norm > 0.0 and u_norm > 0.0) else 1.0
    return w - lr * ratio * u, m_new, v_new, ratio, u


def lamb_step(tensors, step, lr, beta1, beta2, eps, weight_decay):
    """One step over a list of dicts with keys w, g, m, v (and an optional
    per-tensor "weight_decay").  Returns a list of dicts w, m, v, ratio."""
    out = []
    for t in tensors:
        wd = t.get("weight_decay", weight_decay)
        w, m, v, r, _ = lamb_tensor_step(t["w"], t["g"], t["m"], t["v"], step,
                                         lr, beta1, beta2, eps, wd)
        out.append(dict(w=w, m=m, v=v, ratio=r))
    return out


# ZeRO-2 sharding (MegaScale study guide, ch.2 §2.1 parallelism table,
# DP (+ZeRO-2) row: optimizer state and gradients are split over the
# data-parallel ranks).  Each rank holds a contiguous slice of every tensor.
# The step above is elementwise except for the two norms, and a squared
# norm is a sum over elements, so the sharded step is: every rank updates
# its slice of m and v and sums w^2 and u^2 over its slice; the ranks add
# those sums (an all-reduce); every rank forms the same ratio from the
# totals and updates its slice of w.

def lamb_shard_norms(w, g, m, v, step, beta1, beta2, eps, weight_decay):
    """First half on one rank's slice.  Returns (m_new, v_new, sum w^2, sum u^2)."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m_new = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    u = _update(w, m_new, v_new, step, beta1, beta2, eps, weight_decay)
    return m_new, v_new, float(np.sum(w * w)), float(np.sum(u * u))


def lamb_shard_apply(w, m_new, v_new, w_sq_total, u_sq_total, step, lr, beta1, beta2, eps,
                     weight_decay):
    """Second half on one rank's slice, from the norms summed over all ranks.
    Returns (w_new, ratio)."""
    w = np.asarray(w, dtype=np.float64)
    u = _update(w, np.asarray(m_new, dtype=np.float64), np.asarray(v_new, dtype=np.float64),
                step, beta1, beta2, eps, weight_decay)
    ratio = (np.sqrt(w_sq_total) / np.sqrt(u_sq_total)
             if (w_sq_total > 0.0 and u_sq_total > 0.0) else 1.0)
    return w - lr * ratio * u, float(ratio)


def _update(w, m_new, v_new, step, beta1, beta2, eps, weight_decay):
    """u of the published method from the updated moments."""
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    return m_hat / (np.sqrt(v_hat) + eps) + weight_decay * w
