"""Frozen-decision surrogate used to pin the oracle's straight-through backward.

Every rounding decision (rint(u) - u, rint(t2/h) - t2/h), clamp side and
argmax/argmin index is recorded from an exact forward and then held fixed.  The
resulting float64 function of the parameters is smooth, and its exact gradient
is the straight-through gradient (rint replaced by the identity, clamp, max/min,
h and z differentiated exactly), so central finite differences of it check the
hand-written backward term by term.  This is a test pin, not part of the oracle.
"""
from types import SimpleNamespace

import numpy as np

F64 = np.float64


class SmoothOps:
    bf16 = False

    def __init__(self, frozen):
        self.frozen = frozen

    def sigmoid(self, a):
        return 1.0 / (1.0 + np.exp(-np.asarray(a, F64)))

    def to_code(self, x):
        return np.asarray(x, F64)

    def let_act(self, X, s, delta):
        return (np.asarray(X, F64) - np.asarray(delta, F64)[None, :]) / np.asarray(s, F64)[None, :]

    def let_weight(self, W, s):
        return np.asarray(s, F64)[None, :] * np.asarray(W, F64)

    def div(self, X, s):
        return np.asarray(X, F64) / np.asarray(s, F64)[None, :]

    def mul(self, X, s):
        return np.asarray(s, F64)[None, :] * np.asarray(X, F64)

    def quant(self, x, gamma, beta, nbits, key):
        fz = self.frozen[key]
        x = np.asarray(x, F64)
        R = x.shape[0]
        rows = np.arange(R)
        Q = F64(2 ** nbits - 1)
        gamma = np.broadcast_to(np.asarray(gamma, F64), (R,))
        beta = np.broadcast_to(np.asarray(beta, F64), (R,))
        M = x[rows, fz.iM]
        m = x[rows, fz.im]
        t1 = gamma * M
        t2 = beta * m
        h = np.where(fz.floor, 1e-8, (t1 - t2) / Q)
        z = -(t2 / h + fz.rz)
        u = x / h[:, None]
        qmz = np.where(fz.inr, u + fz.r0, fz.q.astype(F64) - z[:, None])
        return SimpleNamespace(Q=Q, gamma=gamma, beta=beta, iM=fz.iM, im=fz.im, M=M, m=m,
                               t1=t1, t2=t2, h=h, floor=fz.floor, z=z, u=u, inr=fz.inr,
                               qmz=qmz, xhat=qmz * h[:, None])

    def act(self, x, abits, key):
        if abits >= 16:
            return None, np.asarray(x, F64)
        st = self.quant(x, 1.0, 1.0, abits, key)
        return st, st.xhat

    def operand(self, a):
        return np.asarray(a, F64)
