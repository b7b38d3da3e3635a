"""Pins of the oracle optimizer and the single-layer calibration loop (CPU only).

* AdamW's first step with |g| >> eps moves each parameter by lr * sign(g); with
  bias correction a constant gradient gives the same step every time.
* AdamW against Adam's closed form on a gradient sequence +g, -g: the second step
  is lr (1 - beta1) / (1 + beta1) in the direction of +g (bias-corrected moments:
  m^ = -(1 - beta1) g / (1 + beta1), v^ = g^2), and weight decay scales theta by
  (1 - lr wd) first.  This pins the update rule for the constants the oracle uses;
  the constants themselves (beta1 0.9, beta2 0.999, eps 1e-8) are not on the pages:
  parity unpinned, a reading (standard defaults).
* SGD is theta - lr g.
* The single-layer fp32 workload (W4A16, LWC only, SGD at lr 5e-3): its logit
  gradients are ~1e-4, so lr * g is about one float32 spacing of the logits at
  4.0: the parameters move by at most a few ulp over the 10 steps and the loss
  barely changes; with a larger step the loss decreases.  The trajectory itself is parity unpinned (the pages give no
  values for it).
"""
import numpy as np

from oracle import linear as ol
from oracle import optim
import synth

F32 = np.float32


def test_adamw_first_step_and_bias_correction():
    rng = np.random.default_rng(0)
    th = rng.standard_normal(100).astype(F32)
    g = (rng.standard_normal(100) * 1e-2).astype(F32)
    m = np.zeros(100, F32)
    v = np.zeros(100, F32)
    t1, m, v = optim.adamw(th, g, m, v, 1, 1e-2)
    assert np.allclose(t1 - th, -1e-2 * np.sign(g), rtol=1e-4, atol=1e-7)
    t2, m, v = optim.adamw(t1, g, m, v, 2, 1e-2)
    assert np.allclose(t2 - t1, t1 - th, rtol=1e-3, atol=1e-7)


def test_adamw_closed_form_two_steps():
    g = np.array([0.3, -2.0, 5e-2], F32)
    th = np.array([1.0, 0.5, -0.25], F32)
    z = np.zeros(3, F32)
    lr = 1e-2
    t1, m, v = optim.adamw(th, g, z, z, 1, lr)
    t2, m, v = optim.adamw(t1, -g, m, v, 2, lr)
    b1, b2, eps = optim.BETA1, optim.BETA2, optim.EPS
    # m^_2 = -(1 - b1) g / (1 + b1) and v^_2 = g^2 exactly; step = -lr m^ / (|g| + eps)
    want = lr * (1 - b1) / (1 + b1) * np.abs(g) / (np.abs(g) + eps) * np.sign(g)
    assert np.allclose(t2.astype(np.float64) - t1, want, rtol=1e-4, atol=2e-8)
    assert np.allclose(m, -(1 - b1) ** 2 * g, rtol=1e-5)
    assert np.allclose(v, (1 - b2) * (1 + b2) * g.astype(np.float64) ** 2, rtol=1e-5)
    # decoupled weight decay: theta (1 - lr wd) - lr m^ / (sqrt(v^) + eps)
    t3, _, _ = optim.adamw(th, g, z, z, 1, lr, weight_decay=0.1)
    assert np.allclose(t3, th * (1 - lr * 0.1) - lr * np.sign(g), rtol=1e-5, atol=1e-7)


def test_sgd():
    th = np.array([1.0, -2.0], F32)
    assert np.allclose(optim.sgd(th, np.array([10.0, 0.0]), 0.1), [0.0, -2.0])


def _run(lr, steps):
    c = synth.LINEAR_CFG1
    inp = synth.linear_inputs(c)
    X, W, B = inp["X"], inp["W"], inp["B"]
    Ystar = ol.reference(X, W, B)
    th0 = ol.init_theta(c.c_in, c.c_out, c.let)
    th = dict(th0)
    losses = []
    for _ in range(steps):
        loss, g, _, _ = ol.calib_step(X, W, B, Ystar, th, c.wbits, c.abits, c.let, bf16=False)
        losses.append(loss)
        th = {k: optim.sgd(th[k], g[k], lr) for k in th}
    return th0, th, losses, g


def test_cfg1_sgd_updates_below_fp32_spacing():
    c = synth.LINEAR_CFG1
    th0, th, losses, g = _run(c.lr_lwc, c.steps)
    spacing = np.spacing(np.float32(4.0))
    assert np.abs(c.lr_lwc * g["a_gamma"]).max() < spacing
    assert all(np.abs(th0[k] - th[k]).max() <= c.steps * spacing for k in th0)
    assert abs(losses[-1] - losses[0]) < 1e-4 * losses[0]


def test_cfg1_sgd_larger_step_decreases_loss():
    th0, th, losses, g = _run(500.0, 10)
    assert losses[-1] < losses[0]
