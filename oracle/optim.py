"""Oracle optimizer updates over the learnable quantization parameters.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows the paper reading "OmniQuant ..." (onecrewdev.com), section "实验证据":
AdamW with zero weight decay, learning rate 5e-3 for the LWC logits and 1e-2 for
the LET parameters, batch size 1.  Adam's beta1 = 0.9, beta2 = 0.999 and
eps = 1e-8 are not on the pages (standard defaults, a reading of a point the
pages leave open).  The single-layer fp32 workload uses plain SGD (lr 5e-3).

Parity: the update rule is pinned by tests/test_oracle_linear.py (first Adam step
is lr * sign(g) for |g| >> eps; Adam's closed form on a +g, -g gradient sequence;
decoupled weight decay; SGD is theta - lr g).  The constants BETA1, BETA2 and EPS
are parity unpinned: the pages give no values, and a different choice would pass
every pin above that does not name them.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

BETA1 = 0.9
BETA2 = 0.999
EPS = 1e-8


def sgd(theta, grad, lr):
    return (np.asarray(theta, F64) - lr * np.asarray(grad, F64)).astype(F32)


def adamw(theta, grad, m, v, step, lr, weight_decay=0.0):
    """One AdamW step (step counts from 1).  Returns (theta, m, v) in float32."""
    th = np.asarray(theta, F64)
    g = np.asarray(grad, F64)
    m = BETA1 * np.asarray(m, F64) + (1.0 - BETA1) * g
    v = BETA2 * np.asarray(v, F64) + (1.0 - BETA2) * g * g
    mhat = m / (1.0 - BETA1 ** step)
    vhat = v / (1.0 - BETA2 ** step)
    th = th * (1.0 - lr * weight_decay) - lr * mhat / (np.sqrt(vhat) + EPS)
    return th.astype(F32), m.astype(F32), v.astype(F32)
