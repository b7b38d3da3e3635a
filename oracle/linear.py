"""Oracle quantized linear layer: forward Y = Q_a(X~) Q_w(W~)^T + B~ and its
straight-through backward (gradients for X, the LWC logits, s and delta).

TEST INFRASTRUCTURE ONLY (see the package header).

Follows the paper reading "OmniQuant ..." (onecrewdev.com), section "LET" (the
linear-layer equation with the quantizers applied to X~ and W~) and section
"LWC" (the weight quantizer).  Weights are stored [C_out x C_in] (Y = X W^T + B),
so the page's s * W scales W's columns.

Operand precision: as ops.ExactOps states (the forward product of a layer with
both quantizers on is exact; other products take the bf16 path's operand casts).

Parity: pinned by tests/test_oracle_linear.py (LET identity with quantizers off,
finite differences of the frozen-decision surrogate, SGD trajectory invariants).
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

from . import quant
from .ops import ExactOps

F32 = np.float32
F64 = np.float64


def forward(X, W, B, theta, wbits, abits, let, ops, group=0):
    """theta: dict with a_gamma, a_beta [C_out] (group-wise LWC: [C_out * C_in /
    group], output-channel major) and (when let) s, delta [C_in]."""
    gamma = ops.sigmoid(theta["a_gamma"])
    beta = ops.sigmoid(theta["a_beta"])
    if let:
        s, delta = theta["s"], theta["delta"]
        Wt = ops.let_weight(W, s)
        Xt = ops.let_act(X, s, delta)
        Bt = quant.bias_fold(W, B, delta)
    else:
        Wt = ops.to_code(W)
        Xt = ops.to_code(X)
        Bt = np.zeros(W.shape[0]) if B is None else np.asarray(B, dtype=F64)
    rows = W.shape[0] * (W.shape[1] // group if group else 1)
    wst = ops.quant(np.reshape(Wt, (rows, -1)), gamma, beta, wbits, "w") if wbits < 16 else None
    ast, Xh = ops.act(Xt, abits, "a")
    Xop = ops.operand(Xh)
    Wop = ops.operand(np.reshape(wst.xhat, np.shape(Wt)) if wst is not None else Wt)
    ep = getattr(ops, "exact_product", None)
    if ep is not None and ep(wbits, abits):
        # both sides quantized: the product of the exact dequantized operands
        Y = np.asarray(Xh, F64) @ np.reshape(wst.xhat, np.shape(Wt)).astype(F64).T
    else:
        Y = Xop @ Wop.T
    Y = Y + Bt[None, :]
    return Y, SimpleNamespace(X=X, W=W, Wt=Wt, Xt=Xt, wst=wst, ast=ast, Xop=Xop, Wop=Wop,
                              gamma=gamma, beta=beta, theta=theta, let=let, ops=ops)


def backward(dY, sv):
    """Gradients of the loss w.r.t. X and theta, given dL/dY."""
    dY = np.asarray(dY, dtype=F64)
    g = {}
    dYo = sv.ops.grad_operand(dY) if hasattr(sv.ops, "grad_operand") else dY
    gXop = dYo @ sv.Wop
    gWop = dYo.T @ sv.Xop
    if sv.wst is None:
        n = np.asarray(sv.theta["a_gamma"]).size
        gWt, g_gamma, g_beta = gWop, np.zeros(n), np.zeros(n)
    else:
        gWt, g_gamma, g_beta = quant.quantize_rows_bwd(np.reshape(gWop, (sv.wst.h.size, -1)),
                                                       sv.wst)
        gWt = np.reshape(gWt, gWop.shape)
    ga = sv.gamma.astype(F64)
    gb = sv.beta.astype(F64)
    g["a_gamma"] = g_gamma * ga * (1.0 - ga)
    g["a_beta"] = g_beta * gb * (1.0 - gb)
    gXt = quant.act_quant_bwd(gXop, sv.ast)
    if sv.let:
        s = np.asarray(sv.theta["s"], dtype=F64)
        W64 = np.asarray(sv.W, dtype=F64)
        Xt = np.asarray(sv.Xt, dtype=F64)
        g["s"] = np.sum(gWt * W64, axis=0) + np.sum(gXt * (-Xt / s[None, :]), axis=0)
        g["delta"] = np.sum(gXt * (-1.0 / s[None, :]), axis=0) + W64.T @ dY.sum(axis=0)
        gX = gXt / s[None, :]
    else:
        gX = gXt
    return gX, g


def reference(X, W, B):
    """The full-precision layer Y* = X W^T + B (float64)."""
    Y = np.asarray(X, dtype=F64) @ np.asarray(W, dtype=F64).T
    if B is not None:
        Y = Y + np.asarray(B, dtype=F64)[None, :]
    return Y


def mse(Y, Ystar):
    """L = mean((Y - Y*)^2) and dL/dY."""
    diff = np.asarray(Y, dtype=F64) - np.asarray(Ystar, dtype=F64)
    return float(np.mean(diff * diff)), 2.0 * diff / diff.size


def init_theta(c_in, c_out, let, a0=4.0):
    th = {"a_gamma": np.full(c_out, a0, F32), "a_beta": np.full(c_out, a0, F32)}
    if let:
        th["s"] = np.ones(c_in, F32)
        th["delta"] = np.zeros(c_in, F32)
    return th


def calib_step(X, W, B, Ystar, theta, wbits, abits, let, bf16, group=0):
    """One fwd + MSE + bwd pass; returns (loss, grads, Y)."""
    Y, sv = forward(X, W, B, theta, wbits, abits, let, ExactOps(bf16), group)
    loss, dY = mse(Y, Ystar)
    _, g = backward(dY, sv)
    return loss, g, Y, sv
