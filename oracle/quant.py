"""Oracle quantizer primitives: LWC weight quantizer, per-token activation
quantizer, LET transforms, and their straight-through backward.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows the paper reading "OmniQuant: Omnidirectionally Calibrated Quantization
for LLMs" (onecrewdev.com):

* section "LWC", the LWC equation: integer codes are the clamp to [0, 2^N - 1] of
  round(W / h) + z, with h = (gamma * max(W) - beta * min(W)) / (2^N - 1) and
  z = -round(beta * min(W) / h); gamma, beta in [0, 1] through a sigmoid.
  Dequantization is (q - z) * h (the tutorial's affine dequantization, section
  2.2, in this convention); gamma = beta = 1 is plain MinMax quantization.
* section "LET", the linear-layer equation: X~ = (X - delta) / s, W~ = s * W
  (s scales W's input channels), B~ = B + delta W; Y = Q_a(X~) Q_w(W~) + B~.
* section "实验证据": weights per output channel, activations per token.

Readings of points the pages leave open:
* rounding ties go to even (IEEE rint);
* h is floored at 1e-8 (a constant row would otherwise divide by zero);
* only the rounding is straight-through (the blog on LWC, section 2.2, states the
  gradient bypasses the rounding); clamp, max/min, h and z are differentiated
  exactly; max/min ties go to the lowest index;
* the activation quantizer is the same asymmetric MinMax with gamma = beta = 1;
* gamma = sigmoid(a) is evaluated in float64 and rounded once to float32.

Parity: pinned by tests/test_oracle_quant.py (worked example, MinMax special
case vs a nearest-grid-point search, brute force over tiny rows, invariants) and
tests/test_oracle_grad.py (finite differences of a frozen-decision surrogate).
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

F32 = np.float32
F64 = np.float64
H_FLOOR = np.float32(1e-8)


def sigmoid32(a) -> np.ndarray:
    """gamma = sigmoid(a): float64 evaluation rounded once to float32."""
    a64 = np.asarray(a, dtype=F64)
    return (1.0 / (1.0 + np.exp(-a64))).astype(F32)


def bf16(a) -> np.ndarray:
    """Round to bf16 (nearest even) through torch's CPU conversion; float64 out.

    float64 input is first rounded to float32 (the GPU holds these tensors in
    float32 before it casts them to bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=F64).astype(F32)))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def quantize_rows(x, gamma, beta, nbits: int) -> SimpleNamespace:
    """Asymmetric N-bit fake quantization of every row of x (float32, exact).

    x: [R, C] float32; gamma, beta: [R] float32 (clipping strengths).
    Returns the state the backward needs plus codes and dequantized values.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    R, C = x.shape
    gamma = np.broadcast_to(np.asarray(gamma, dtype=F32), (R,))
    beta = np.broadcast_to(np.asarray(beta, dtype=F32), (R,))
    Q = F32(2 ** nbits - 1)
    rows = np.arange(R)
    iM = np.argmax(x, axis=1)           # first index of the maximum
    im = np.argmin(x, axis=1)           # first index of the minimum
    M = x[rows, iM]
    m = x[rows, im]
    t1 = gamma * M                      # fl32(gamma * max)
    t2 = beta * m                       # fl32(beta * min)
    h = (t1 - t2) / Q                   # fl32(fl32(t1 - t2) / Q)
    floor = h < H_FLOOR
    h = np.where(floor, H_FLOOR, h).astype(F32)
    zq = t2 / h                         # fl32(t2 / h)
    z = -np.rint(zq)
    u = x / h[:, None]                  # fl32(x / h)
    ru = np.rint(u)
    r = ru + z[:, None]
    inr = (r >= 0) & (r <= Q)
    q = np.clip(r, F32(0), Q)
    qmz = q - z[:, None]                # exact small integers
    xhat = qmz * h[:, None]             # fl32((q - z) * h)
    return SimpleNamespace(
        nbits=nbits, Q=Q, x=x, gamma=gamma, beta=beta, iM=iM, im=im, M=M, m=m,
        t1=t1, t2=t2, h=h, floor=floor, z=z, u=u, inr=inr, q=q, qmz=qmz, xhat=xhat,
        codes=q.astype(np.uint8),
        # residuals of the rounding decisions (used only to build the smooth
        # surrogate that pins the backward by finite differences)
        r0=ru.astype(F64) - u.astype(F64), rz=np.rint(zq).astype(F64) - zq.astype(F64))


def quantize_rows_bwd(g, st) -> tuple:
    """Straight-through backward of ``quantize_rows``.

    g: upstream gradient w.r.t. xhat [R, C].  Returns (g_x [R, C], g_gamma [R],
    g_beta [R]) in float64.  Only rint is replaced by the identity; the clamp
    contributes its indicator, h and z their exact derivatives, max/min a
    one-hot at the (first) argmax/argmin.
    """
    g = np.asarray(g, dtype=F64)
    R = g.shape[0]
    rows = np.arange(R)
    h = st.h.astype(F64)
    Q = F64(st.Q)
    inr = st.inr
    u = st.u.astype(F64)
    qmz = st.qmz.astype(F64)
    t2 = st.t2.astype(F64)
    gamma = st.gamma.astype(F64)
    beta = st.beta.astype(F64)
    M = st.M.astype(F64)
    m = st.m.astype(F64)
    # d xhat / d h = (q - z) - in * x / h ;  d xhat / d z = -h (1 - in)
    g_h = np.sum(g * (qmz - inr * u), axis=1)
    g_z = np.sum(g * (1.0 - inr), axis=1) * (-h)
    # z = -round(t2 / h): dz/dt2 = -1/h, dz/dh = t2 / h^2 (rint straight through)
    G = np.where(st.floor, 0.0, g_h + g_z * t2 / (h * h))
    g_t1 = G / Q
    g_t2 = -G / Q - g_z / h
    g_gamma = g_t1 * M
    g_beta = g_t2 * m
    g_M = g_t1 * gamma
    g_m = g_t2 * beta
    gx = g * inr
    np.add.at(gx, (rows, st.iM), g_M)
    np.add.at(gx, (rows, st.im), g_m)
    return gx, g_gamma, g_beta


def act_quant(x, abits: int):
    """Per-token (row) asymmetric MinMax quantizer; abits >= 16 is a pass-through."""
    x = np.ascontiguousarray(x, dtype=F32)
    if abits >= 16:
        return None, x
    st = quantize_rows(x, F32(1), F32(1), abits)
    return st, st.xhat


def act_quant_bwd(g, st):
    if st is None:
        return np.asarray(g, dtype=F64)
    return quantize_rows_bwd(g, st)[0]


def let_act(X, s, delta) -> np.ndarray:
    """X~ = (X - delta) / s, float32, two rounded ops (no FMA)."""
    X = np.asarray(X, dtype=F32)
    return (X - np.asarray(delta, dtype=F32)[None, :]) / np.asarray(s, dtype=F32)[None, :]


def let_weight(W, s) -> np.ndarray:
    """W~ = s * W with s over W's input channels (columns), float32."""
    return np.asarray(s, dtype=F32)[None, :] * np.asarray(W, dtype=F32)


def bias_fold(W, B, delta) -> np.ndarray:
    """B~ = B + delta W (W is [C_out x C_in], so the sum runs over C_in), float64."""
    out = np.asarray(W, dtype=F64) @ np.asarray(delta, dtype=F64)
    if B is not None:
        out = out + np.asarray(B, dtype=F64)
    return out


def group_rows(Wt, group):
    """[C_out, C_in] -> [C_out * C_in / group, group]: each output channel split into
    groups of `group` consecutive input channels, one quantizer row per group
    (group-wise LWC: clipping strengths, step and zero point per group)."""
    Wt = np.asarray(Wt)
    C_out, C_in = Wt.shape
    assert C_in % group == 0, (C_in, group)
    return Wt.reshape(C_out * (C_in // group), group)


def lwc_fakequant(W, a_gamma, a_beta, nbits, s=None, delta=None, B=None, group=None):
    """The weight side of one linear layer: LET on W, LWC, bias fold.

    group: None (or C_in) quantizes each output channel as one row; otherwise each
    run of `group` input channels of an output channel is its own row, with its
    own logits: a_gamma / a_beta are [C_out * C_in / group], output-channel major.
    Codes and W_hat keep the [C_out, C_in] shape; h, z and st are per group."""
    Wt = let_weight(W, s) if s is not None else np.asarray(W, dtype=F32)
    C_out, C_in = Wt.shape
    g = C_in if group is None else int(group)
    st = quantize_rows(group_rows(Wt, g), sigmoid32(a_gamma), sigmoid32(a_beta), nbits)
    Bt = bias_fold(W, B, delta) if delta is not None else (
        np.zeros(W.shape[0]) if B is None else np.asarray(B, dtype=F64))
    return SimpleNamespace(Wt=Wt, st=st, W_hat=st.xhat.reshape(C_out, C_in),
                           codes=st.codes.reshape(C_out, C_in), h=st.h, z=st.z,
                           B_tilde=Bt, group=g)


def code_product(qa, h_a, z_a, qb, h_b, z_b, bias=None) -> np.ndarray:
    """The quantized product Y = Q_a(X~) Q_w(W~)^T + B~ (section "LET") written on
    the integer codes: each operand row r holds (q_r - z_r) h_r (section "LWC",
    dequantization), so Y = ((qa - z_a) h_a) ((qb - z_b) h_b)^T + bias, float64.
    qa [M, K], qb [N, K] codes; h_*, z_* per row; bias [N] or None."""
    A = (np.asarray(qa, dtype=F64) - np.asarray(z_a, dtype=F64)[:, None]) * \
        np.asarray(h_a, dtype=F64)[:, None]
    B = (np.asarray(qb, dtype=F64) - np.asarray(z_b, dtype=F64)[:, None]) * \
        np.asarray(h_b, dtype=F64)[:, None]
    out = A @ B.T
    if bias is not None:
        out = out + np.asarray(bias, dtype=F64)[None, :]
    return out


def lwc_bwd(g_What, ref):
    """Straight-through backward of ``lwc_fakequant`` (result ``ref``) for the
    upstream gradient w.r.t. W_hat: returns (dL/dW~ [C_out, C_in], dL/dgamma,
    dL/dbeta), the last two per quantizer row (output channel or group)."""
    g_What = np.asarray(g_What, F64)
    gx, gg, gb = quantize_rows_bwd(group_rows(g_What, ref.group), ref.st)
    return gx.reshape(g_What.shape), gg, gb
