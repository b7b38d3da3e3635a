"""Finite-difference pins of the oracle's hand-written straight-through backward.

The forward is re-evaluated in float64 with every discrete decision frozen
(tests/smooth_surrogate.py); that function is smooth and its exact gradient is
the straight-through gradient, so central differences must match the oracle's
backward for every parameter group: LWC logits, LET s / delta, s_a, and the
layer input.  A dropped term, a wrong sign or a transposed operand anywhere in
the backward fails one of these.
"""
import copy

import numpy as np
import pytest

from oracle import block as ob
from oracle import linear as ol
from oracle import quant
from oracle.ops import ExactOps
from smooth_surrogate import SmoothOps
import synth

F32 = np.float32
F64 = np.float64


def _fd(loss_fn, theta, grads, names, rng, n=5, eps=1e-6, rtol=2e-5):
    worst = 0.0
    for name in names:
        g = np.asarray(grads[name], F64).reshape(-1)
        scale = max(np.abs(g).max(), 1e-300)
        idx = rng.choice(g.size, size=min(n, g.size), replace=False)
        for i in idx:
            tp = copy.deepcopy(theta)
            tm = copy.deepcopy(theta)
            tp[name].reshape(-1)[i] += eps
            tm[name].reshape(-1)[i] -= eps
            fd = (loss_fn(tp) - loss_fn(tm)) / (2 * eps)
            err = abs(fd - g[i]) / scale
            worst = max(worst, err)
            assert err < rtol, (name, i, fd, g[i], scale)
        assert np.abs(g).max() > 0, name
    return worst


def test_quantizer_rows_fd():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((6, 40)) * 0.5).astype(F32)
    gamma = rng.uniform(0.6, 1.0, 6).astype(F32)
    beta = rng.uniform(0.6, 1.0, 6).astype(F32)
    ex = quant.quantize_rows(x, gamma, beta, 3)
    frozen = {"k": ex}
    ops = SmoothOps(frozen)
    w = rng.standard_normal(x.shape)

    def L(p):
        st = ops.quant(p["x"], p["gamma"], p["beta"], 3, "k")
        return float(np.sum(w * st.xhat))

    p0 = {"x": x.astype(F64), "gamma": gamma.astype(F64), "beta": beta.astype(F64)}
    st = ops.quant(p0["x"], p0["gamma"], p0["beta"], 3, "k")
    gx, gg, gb = quant.quantize_rows_bwd(w, st)
    assert np.any(~st.inr)  # clipping is exercised
    _fd(L, p0, {"x": gx, "gamma": gg, "beta": gb}, ["x", "gamma", "beta"], rng, n=12)


@pytest.mark.parametrize("abits,let,group", [(4, True, 0), (16, True, 0), (8, False, 0),
                                             (4, True, 8), (16, False, 8)])
def test_linear_fd(abits, let, group):
    rng = np.random.default_rng(1)
    c = synth.reduced(synth.LINEAR_CFG1, T=12, c_in=24, c_out=10)
    inp = synth.linear_inputs(c)
    X, W, B = inp["X"], inp["W"], inp["B"] + rng.standard_normal(10).astype(F32)
    th = ol.init_theta(24, 10, let)
    rows = 10 * (24 // group if group else 1)
    th["a_gamma"] = rng.uniform(0.5, 4.0, rows).astype(F32)
    th["a_beta"] = rng.uniform(0.5, 4.0, rows).astype(F32)
    if let:
        th["s"] = rng.uniform(0.5, 2.0, 24).astype(F32)
        th["delta"] = (rng.standard_normal(24) * 0.3).astype(F32)
    Ystar = ol.reference(X, W, B)
    ex = ExactOps(bf16=False)
    ol.forward(X, W, B, th, 4, abits, let, ex, group)
    ops = SmoothOps(ex.states)
    th64 = {k: v.astype(F64) for k, v in th.items()}
    th64["X"] = X.astype(F64)

    def L(p):
        Y, _ = ol.forward(p["X"], W, B, p, 4, abits, let, ops, group)
        return ol.mse(Y, Ystar)[0]

    Y, sv = ol.forward(th64["X"], W, B, th64, 4, abits, let, ops, group)
    loss, dY = ol.mse(Y, Ystar)
    gX, g = ol.backward(dY, sv)
    g["X"] = gX
    names = ["a_gamma", "a_beta", "X"] + (["s", "delta"] if let else [])
    _fd(L, th64, g, names, rng, n=6)


def _tiny_block(ffn_only=False, n_q=4, n_kv=2, wbits=4, abits=4, group=0):
    return synth.BlockCfg(cfg=4, T=7, d=16, n_q=n_q, n_kv=n_kv, F=24, wbits=wbits,
                          abits=abits, head_dim=8, ffn_only=ffn_only, n_out=2,
                          out_lo=5.0, out_hi=10.0, group=group)


@pytest.mark.parametrize("kind", ["mha_w4a4", "gqa_w4a4", "gqa_w4a16", "ffn_w3a16", "mha_w16a4",
                                  "mha_w4a4_g8", "ffn_w3a16_g8"])
def test_block_fd(kind):
    c = {"mha_w4a4": _tiny_block(n_q=2, n_kv=2),
         "gqa_w4a4": _tiny_block(n_q=4, n_kv=2),
         "gqa_w4a16": _tiny_block(n_q=4, n_kv=2, abits=16),
         "ffn_w3a16": _tiny_block(ffn_only=True, wbits=3, abits=16),
         "mha_w16a4": _tiny_block(n_q=2, n_kv=2, wbits=16, abits=4),
         # group-wise LWC: 8 input channels per clipping group
         "mha_w4a4_g8": _tiny_block(n_q=2, n_kv=2, group=8),
         "ffn_w3a16_g8": _tiny_block(ffn_only=True, wbits=3, abits=16, group=8)}[kind]
    rng = np.random.default_rng(5)
    inp = synth.block_inputs(c)
    # larger weights than N(0, 0.02^2) so the tiny block is far from linear
    Wd = {k: (v * 10).astype(F32) for k, v in inp.items() if k.startswith("W_")}
    x = inp["x"]
    shapes = synth.block_weight_shapes(c)
    th = ob.init_theta(c, shapes)
    for k in th:
        if k.startswith("a_"):
            th[k] = rng.uniform(0.5, 4.0, th[k].size).astype(F32)
        elif k.startswith("s"):
            th[k] = rng.uniform(0.6, 1.6, th[k].size).astype(F32)
        else:
            th[k] = (rng.standard_normal(th[k].size) * 0.2).astype(F32)
    ystar = ob.reference(c, x, Wd) + rng.standard_normal((c.T, c.d)) * 0.3
    ex = ExactOps(bf16=False)
    ob.forward(c, x, Wd, th, ex)
    ops = SmoothOps(ex.states)
    th64 = {k: v.astype(F64) for k, v in th.items()}

    def L(p):
        y, _ = ob.forward(c, x, Wd, p, ops)
        return ob.mse(y, ystar)[0]

    loss, g, y, S = ob.calib_step(c, x, Wd, ystar, th64, ops)
    names = [n for n, _ in ob.theta_layout(c, shapes)]
    if c.wbits >= 16:
        names = [n for n in names if not n.startswith("a_")]
        for n in th:
            if n.startswith("a_"):
                assert np.all(g[n] == 0)
    _fd(L, th64, g, names, rng, n=4)
