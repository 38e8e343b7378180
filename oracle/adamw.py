"""fp64 AdamW step over a flat buffer of parameters (test infrastructure: see
oracle/__init__.py for who may use it).

The oreateai.com Megatron-LM analysis ("In-Depth Analysis of Distributed Training
Frameworks for Large Models ... Megatron-LM"), section 2.2, reports a fused AdamW
optimizer step (one kernel instead of PyTorch's separate element-wise operations) and
lists beta1 = 0.9, beta2 = 0.95 in section 3.1. It does not spell the update out; the
reading taken here is the textbook one: Adam's moment estimates with bias correction
(Kingma and Ba, "Adam: A Method for Stochastic Optimization", Algorithm 1) and weight
decay decoupled from the gradient (Loshchilov and Hutter, "Decoupled Weight Decay
Regularization", AdamW), applied to the fp32 master parameters. grad_scale multiplies
the gradient first (the inverse of a loss scale, or a clipping factor).

Pins (tests/test_oracle_adamw.py): closed forms of the first step from zero moments,
of a constant gradient (bias correction makes every step the same), of decay alone,
Adam's invariance to the gradient's scale, and torch.optim.AdamW in fp64 on the CPU.
"""
from __future__ import annotations

import numpy as np


def adamw_step(p, g, m, v, *, lr, beta1, beta2, eps, weight_decay, step, grad_scale=1.0):
    """One AdamW step at step number `step` (1-based). Returns (p, m, v) in float64."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64) * grad_scale
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    # exponential moving averages of the gradient and of its square
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * g * g
    # bias-corrected estimates (the averages start at zero)
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    # decoupled weight decay on the current parameters, then the Adam step
    p_new = p - lr * weight_decay * p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m_new, v_new
