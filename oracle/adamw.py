"""AdamW on the adapter parameters (Loshchilov & Hutter 2019, decoupled weight decay).

The pages are silent on the optimizer; the reading taken is the common
PyTorch form: p <- p (1 - lr wd); m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
p <- p - lr * (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps).
The float master parameter is updated; the bf16 working copy is rnd(p).
"""
import numpy as np


def adamw_step(p, g, m, v, step, lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0):
    """One step (step counts from 1). Returns new (p, m, v)."""
    p = p * (1.0 - lr * wd)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    p = p - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v
