"""Oracle of the sequential multi-block calibration.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows the paper reading "OmniQuant: ..." (onecrewdev.com):
* section "框架", the block-wise objective: block k's loss compares the
  full-precision block F(W, X) with the quantized block F(Q_w(W), Q_a(X)) on the
  same input X;
* the sentence after it and the flowchart: blocks are processed in order; once block
  k is calibrated (frozen), its quantized weights compute block k+1's input;
* section "实验证据": batch size 1, a number of epochs over the calibration samples,
  AdamW with zero weight decay, learning rate 5e-3 for the LWC logits and 1e-2 for
  the LET parameters.

Readings of points the pages leave open:
* "the same input X" is the quantized chain's input (there is no separate
  full-precision chain): the target of block k is F(W_k, X_k) with X_k the output of
  the calibrated blocks 1..k-1;
* the targets are computed once per block, before its first step (the weights and
  inputs do not change while the block is calibrated);
* block inputs are bf16 (a block's fp32/float64 output is rounded to bf16 before it
  becomes the next input), as the hidden state of a half-precision model;
* each block starts from the initial parameters (logits a0, s = 1, delta = 0,
  s_a = 1) with zero AdamW moments and its own step count from 1;
* within an epoch the samples are taken in their stored order.

Parity: pinned by tests/test_oracle_driver.py (the schedule, the chaining of
inputs and targets through the stack, the reduction to the one-block step, and the
loss falling over the epochs).
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

from . import block as ob
from . import optim, quant
from .ops import ExactOps

F32 = np.float32
F64 = np.float64


def step(c, shapes, Wd, x, ystar, vec, m, v, t, ops=None):
    """One calibration step at batch size 1 (step count t from 1): forward, MSE,
    backward, then AdamW with lr_lwc on the clipping logits and lr_let on the rest.
    Returns (vec, m, v, loss, grad vector)."""
    th = ob.unpack(c, shapes, vec)
    loss, g, _, _ = ob.calib_step(c, x, Wd, ystar, th, ops or ExactOps(bf16=True))
    gv = ob.pack(c, shapes, g)
    n_lwc = sum(n for name, n in ob.theta_layout(c, shapes) if name.startswith("a_"))
    out = []
    for sl, lr in ((slice(0, n_lwc), c.lr_lwc), (slice(n_lwc, vec.size), c.lr_let)):
        out.append(optim.adamw(vec[sl], gv[sl], m[sl], v[sl], t, lr, 0.0))   # zero weight decay
    vec2 = np.concatenate([o[0] for o in out])
    m2 = np.concatenate([o[1] for o in out])
    v2 = np.concatenate([o[2] for o in out])
    return vec2, m2, v2, loss, gv


def targets(c, Wd, xs):
    """Full-precision block outputs on the block's current inputs (float64)."""
    return [ob.reference(c, x, Wd) for x in xs]


def next_inputs(c, Wd, vec, xs, ops=None):
    """The calibrated block's quantized outputs, rounded to bf16."""
    shapes = _shapes(c)
    th = ob.unpack(c, shapes, vec)
    return [quant.bf16(ob.forward(c, x, Wd, th, ops or ExactOps(bf16=True))[0]) for x in xs]


def _shapes(c):
    """[C_out, C_in] of the block's linears (q, k, v, o, gate, up, down)."""
    dq, dk = c.n_q * c.head_dim, c.n_kv * c.head_dim
    return {"q": (dq, c.d), "k": (dk, c.d), "v": (dk, c.d), "o": (c.d, dq),
            "gate": (c.F, c.d), "up": (c.F, c.d), "down": (c.d, c.F)}


def calibrate(c, blocks, samples, epochs, a0=4.0, ops=None, on_step=None):
    """blocks: list of weight dicts {W_q, ..., W_down}; samples: list of [T, d]
    (bf16 values).  on_step(SimpleNamespace(block, epoch, sample, step, loss)).
    Returns (per-block parameter vectors, final inputs, per-block losses [epochs, n])."""
    shapes = _shapes(c)
    xs = [quant.bf16(np.asarray(s, F64)) for s in samples]
    vecs, losses = [], []
    for b, Wd in enumerate(blocks):
        ys = targets(c, Wd, xs)
        vec = ob.pack(c, shapes, ob.init_theta(c, shapes, a0))
        m = np.zeros_like(vec)
        v = np.zeros_like(vec)
        t = 0
        L = np.zeros((epochs, len(xs)))
        for e in range(epochs):
            for i in range(len(xs)):
                t += 1
                vec, m, v, L[e, i], _ = step(c, shapes, Wd, xs[i], ys[i], vec, m, v, t, ops)
                if on_step is not None:
                    on_step(SimpleNamespace(block=b, epoch=e, sample=i, step=t, loss=L[e, i]))
        vecs.append(vec)
        losses.append(L)
        xs = next_inputs(c, Wd, vec, xs, ops)
    return vecs, xs, losses
