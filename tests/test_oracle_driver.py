"""Pins of the multi-block calibration oracle (oracle/driver.py).

* schedule: batch size 1, epochs over the samples in order, the step count
  restarting at 1 in every block (paper reading, section "实验证据");
* a block whose weights are all zero is exactly the identity (attention output and
  FFN output are 0 for the full-precision and the quantized block alike, so its
  loss and gradient are 0 and AdamW leaves its parameters alone); a stack with such
  a block in front must reproduce the one-block calibration of the block behind it
  bit for bit, and one behind it must pass the quantized outputs through;
* the one-block, one-sample, one-epoch run is one calibration step of the block
  (pinned by test_oracle_block / test_oracle_grad) followed by AdamW (pinned by
  its closed form in test_oracle_linear);
* the target of block k is the full-precision block on block k's input taken from
  the quantized chain (the objective of section "框架" has the same X in both terms),
  not on a separate full-precision chain;
* calibration lowers the loss over the epochs (the purpose of the method).
"""
import numpy as np
import pytest

import synth
from oracle import block as ob
from oracle import driver as od
from oracle import optim
from oracle.ops import ExactOps

F64 = np.float64


def tiny(base, **kw):
    args = dict(T=64, d=256, n_q=2, n_kv=2, F=512, n_out=3)
    args.update(kw)
    return synth.reduced(base, **args)


def zero_block(c):
    return {k: np.zeros(s, np.float32) for k, s in
            (("W_" + n, sh) for n, sh in synth.block_weight_shapes(c).items())}


def test_schedule():
    c = tiny(synth.BLOCK_CFG4_W2G128, T=32)
    blocks, xs = synth.stack_inputs(c, 2, 3)
    seen = []
    od.calibrate(c, blocks, list(xs), 2, on_step=lambda s: seen.append(
        (s.block, s.epoch, s.sample, s.step)))
    want = [(b, e, i, e * 3 + i + 1) for b in range(2) for e in range(2) for i in range(3)]
    assert seen == want


@pytest.mark.parametrize("base", [synth.BLOCK_CFG4, synth.BLOCK_CFG4_W2G128])
def test_zero_block_in_front_is_transparent(base):
    c = tiny(base)
    blocks, xs = synth.stack_inputs(c, 1, 2)
    v1, x1, L1 = od.calibrate(c, blocks, list(xs), 2)
    v2, x2, L2 = od.calibrate(c, [zero_block(c)] + blocks, list(xs), 2)
    shapes = synth.block_weight_shapes(c)
    assert np.array_equal(v2[0], ob.pack(c, shapes, ob.init_theta(c, shapes)))
    assert np.all(L2[0] == 0.0)
    assert np.array_equal(v2[1], v1[0])
    assert np.array_equal(L2[1], L1[0])
    for a, b in zip(x1, x2):
        assert np.array_equal(a, b)


def test_zero_block_behind_passes_outputs():
    c = tiny(synth.BLOCK_CFG4)
    blocks, xs = synth.stack_inputs(c, 1, 2)
    v1, x1, _ = od.calibrate(c, blocks, list(xs), 1)
    v2, x2, _ = od.calibrate(c, blocks + [zero_block(c)], list(xs), 1)
    assert np.array_equal(v2[0], v1[0])
    for a, b in zip(x1, x2):
        assert np.array_equal(a, b)


def test_one_step_is_block_step_then_adamw():
    c = tiny(synth.BLOCK_CFG4)
    blocks, xs = synth.stack_inputs(c, 1, 1)
    vecs, _, L = od.calibrate(c, blocks, list(xs), 1)
    shapes = synth.block_weight_shapes(c)
    th0 = ob.init_theta(c, shapes)
    x = xs[0].astype(F64)
    loss, g, _, _ = ob.calib_step(c, x, blocks[0], ob.reference(c, x, blocks[0]), th0,
                                  ExactOps(bf16=True))
    assert L[0][0, 0] == loss
    for name, _ in ob.theta_layout(c, shapes):
        lr = c.lr_lwc if name.startswith("a_") else c.lr_let
        z = np.zeros_like(th0[name])
        # the gradient is held as the packed float32 vector
        want = optim.adamw(th0[name], g[name].astype(np.float32), z, z, 1, lr)[0]
        got = ob.unpack(c, shapes, vecs[0])[name]
        assert np.array_equal(got, want), name


def test_target_uses_quantized_chain():
    """Block 2's first loss: its quantized forward on the quantized chain's input
    against the full-precision block on that same input.  A separate
    full-precision chain would give another value (the W2 block 1 moves the
    quantized chain well away from it)."""
    c = tiny(synth.BLOCK_CFG4_W2G128)
    blocks, xs = synth.stack_inputs(c, 2, 1)
    firsts = {}
    od.calibrate(c, blocks, list(xs), 1,
                 on_step=lambda s: firsts.setdefault(s.block, s.loss))
    shapes = synth.block_weight_shapes(c)
    v1 = od.calibrate(c, blocks[:1], list(xs), 1)[0][0]
    th = ob.unpack(c, shapes, v1)
    y_q = ob.forward(c, xs[0].astype(F64), blocks[0], th, ExactOps(bf16=True))[0]
    x_q = synth.to_bf16(y_q.astype(np.float32)).astype(F64)
    init = ob.init_theta(c, shapes)
    y2, _ = ob.forward(c, x_q, blocks[1], init, ExactOps(bf16=True))
    want, _ = ob.mse(y2, ob.reference(c, x_q, blocks[1]))
    assert firsts[1] == pytest.approx(want, rel=1e-12)
    # the mistaken reading (training on the quantized chain's input against a target
    # from a separate full-precision chain) gives a measurably different loss
    x_fp = synth.to_bf16(ob.reference(c, xs[0].astype(F64), blocks[0]).astype(np.float32))
    other, _ = ob.mse(y2, ob.reference(c, x_fp.astype(F64), blocks[1]))
    assert abs(other - want) > 0.05 * want


@pytest.mark.parametrize("base", [synth.BLOCK_CFG4, synth.BLOCK_CFG4_W2G128])
def test_loss_falls(base):
    c = tiny(base)
    blocks, xs = synth.stack_inputs(c, 2, 2)
    _, _, L = od.calibrate(c, blocks, list(xs), 8)
    for Lb in L:
        # the W4A4 curve is noisy at this size: the best of the last three epochs
        assert Lb[-3:].mean(axis=1).min() < 0.96 * Lb[0].mean()
