"""AdamW step on the LoRA matrices, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[rkmt] §3.5 and [czcl] §3.2 train the adapter with AdamW (paged, 8- or
32-bit states, learning rate 2e-4); only A and B carry optimizer state
([kwkr] §2.3: the 4-bit weight gets no gradient).  The paging is a host
memory feature and out of this path; the step itself is the published
AdamW with decoupled weight decay (Loshchilov and Hutter), restated here in
the order a fused kernel applies it:

    p <- p (1 - lr wd)
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

with 32-bit states (the reading of "32bit" on the pages).
"""

import numpy as np


def adamw_step(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW step; returns (p, m, v) as new fp64 arrays."""
    if step < 1:
        raise ValueError("oracle: step counts from 1")
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * weight_decay)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
