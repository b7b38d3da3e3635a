"""GPU parity of the quantized linear layer (forward, MSE, straight-through
backward, optimizer) against the CPU oracle, through the C ABI.

* single fp32 layer, W4A16, LWC only, 10 SGD steps (fp32 path; 1e-4 relative);
* the attention projection, bf16, W4A4 with LWC + LET, at a ragged reduced size
  and at its full 2048 x 4096 x 4096 size (bf16 path; 2e-2 relative).
"""
import numpy as np
import pytest
import torch

import post_quantization_amd as omq
from oracle import linear as ol
from oracle import optim
import synth
from gpu_util import DEV, dev, host, log, rel

pytestmark = pytest.mark.gpu

F32 = np.float32


def _theta_vec(th, let):
    parts = [th["a_gamma"], th["a_beta"]] + ([th["s"], th["delta"]] if let else [])
    return np.concatenate(parts).astype(F32)


def _split(vec, c_in, rows, let):
    out = {"a_gamma": vec[:rows], "a_beta": vec[rows:2 * rows]}
    if let:
        out["s"] = vec[2 * rows:2 * rows + c_in]
        out["delta"] = vec[2 * rows + c_in:]
    return out


def _run_gpu(c, X, W, B, Ystar, theta_vec, group=0):
    bf = not c.fp32
    tdt = torch.bfloat16 if bf else torch.float32
    d = omq.QLinearDesc(c.T, c.c_in, c.c_out, c.wbits, c.abits, c.let,
                        omq.PATH_BF16 if bf else omq.PATH_FP32, group)
    ws = torch.empty(omq.qlinear_workspace_size(d), dtype=torch.uint8, device=DEV)
    tX, tW, tB = dev(X, tdt), dev(W, tdt), dev(B)
    th = dev(theta_vec)
    Y = torch.empty(c.T, c.c_out, dtype=torch.float32, device=DEV)
    omq.qlinear_fwd(d, tX, tW, tB, th, Y, ws)
    tYs = dev(Ystar)
    diff = Y - tYs
    loss = float((diff * diff).mean())
    dY = (2.0 / diff.numel()) * diff
    dX = torch.empty(c.T, c.c_in, dtype=torch.float32, device=DEV)
    dth = torch.empty_like(th)
    omq.qlinear_bwd(d, tX, tW, th, dY.contiguous(), dX, dth, ws)
    torch.cuda.synchronize()
    return host(Y), loss, host(dX), host(dth)


def test_cfg1_fp32_sgd_trajectory():
    c = synth.LINEAR_CFG1
    inp = synth.linear_inputs(c)
    X, W, B = inp["X"], inp["W"], inp["B"]
    Ystar = ol.reference(X, W, B)
    th = ol.init_theta(c.c_in, c.c_out, c.let)
    vec = _theta_vec(th, c.let)
    for step in range(c.steps):
        Yg, lg, dXg, dthg = _run_gpu(c, X, W, B, Ystar, vec)
        loss, g, Y, sv = ol.calib_step(X, W, B, Ystar, th, c.wbits, c.abits, c.let, bf16=False)
        gX, _ = ol.backward(2 * (Y - Ystar) / Y.size, sv)
        log("cfg1 step", step, lg, loss)
        assert rel(Yg, Y) < 1e-5
        assert abs(lg - loss) <= 1e-4 * loss
        assert rel(dthg, _theta_vec(g, c.let)) < 1e-4
        assert rel(dXg, gX) < 1e-4
        th = {k: optim.sgd(th[k], g[k], c.lr_lwc) for k in th}
        vec = _theta_vec(th, c.let)


@pytest.mark.parametrize("size", ["ragged", "full"])
def test_cfg2_bf16_w4a4_let(size):
    c = synth.LINEAR_CFG2
    if size == "ragged":
        c = synth.reduced(c, T=264, c_in=520, c_out=392, n_out=6)
    log("cfg2", size, c.T, c.c_in, c.c_out)
    inp = synth.linear_inputs(c)
    X, W, B = inp["X"], inp["W"], inp["B"]
    rng = np.random.default_rng(21)
    th = ol.init_theta(c.c_in, c.c_out, True)
    th["a_gamma"] = rng.uniform(2.0, 5.0, c.c_out).astype(F32)
    th["a_beta"] = rng.uniform(2.0, 5.0, c.c_out).astype(F32)
    th["s"] = rng.uniform(0.7, 1.4, c.c_in).astype(F32)
    th["delta"] = (rng.standard_normal(c.c_in) * 0.05).astype(F32)
    Ystar = ol.reference(X, W, B)
    Yg, lg, dXg, dthg = _run_gpu(c, X, W, B, Ystar, _theta_vec(th, True))
    loss, g, Y, sv = ol.calib_step(X, W, B, Ystar, th, c.wbits, c.abits, True, bf16=True)
    gX, _ = ol.backward(2 * (Y - Ystar) / Y.size, sv)
    log("loss gpu", lg, "oracle", loss)
    assert rel(Yg, Y) < 1e-4
    assert abs(lg - loss) <= 2e-2 * loss
    gsplit = _split(dthg, c.c_in, c.c_out, True)
    for k in ("a_gamma", "a_beta", "s", "delta"):
        e = rel(gsplit[k], g[k])
        log("grad", k, e)
        assert e < 2e-2, k
    assert rel(dXg, gX) < 2e-2


@pytest.mark.parametrize("path,wbits", [("bf16", 3), ("fp32", 2)])
def test_group128_lwc_linear(path, wbits):
    """Group-wise LWC (128 input channels per clipping group) with LET, weight-only:
    forward, loss and every gradient against the oracle, on both paths (bf16: the
    group state read per 128-column tile inside the fused dW epilogue; fp32: the
    grouped tile pass)."""
    fp32 = path == "fp32"
    c = synth.reduced(synth.LINEAR_CFG2, T=256, c_in=640, c_out=264, n_out=6, wbits=wbits,
                      abits=16, fp32=fp32)
    log("g128 linear", path, wbits)
    inp = synth.linear_inputs(c)
    X, W, B = inp["X"], inp["W"], inp["B"]
    rng = np.random.default_rng(31)
    rows = c.c_out * (c.c_in // 128)
    th = ol.init_theta(c.c_in, c.c_out, True)
    th["a_gamma"] = rng.uniform(2.0, 5.0, rows).astype(F32)
    th["a_beta"] = rng.uniform(2.0, 5.0, rows).astype(F32)
    th["s"] = rng.uniform(0.7, 1.4, c.c_in).astype(F32)
    th["delta"] = (rng.standard_normal(c.c_in) * 0.05).astype(F32)
    Ystar = ol.reference(X, W, B)
    Yg, lg, dXg, dthg = _run_gpu(c, X, W, B, Ystar, _theta_vec(th, True), group=128)
    loss, g, Y, sv = ol.calib_step(X, W, B, Ystar, th, c.wbits, c.abits, True, bf16=not fp32,
                                   group=128)
    gX, _ = ol.backward(2 * (Y - Ystar) / Y.size, sv)
    tol = 1e-4 if fp32 else 2e-2
    log("loss gpu", lg, "oracle", loss)
    assert rel(Yg, Y) < (1e-5 if fp32 else 1e-4)
    assert abs(lg - loss) <= tol * loss
    gsplit = _split(dthg, c.c_in, rows, True)
    for k in ("a_gamma", "a_beta", "s", "delta"):
        e = rel(gsplit[k], g[k])
        log("grad", k, e)
        assert e < tol, k
    assert rel(dXg, gX) < tol
