"""GPU parity of the sequential multi-block calibration (post_quantization_amd.driver)
against the oracle (oracle/driver.py), through the C ABI.

A run of several steps drifts apart from the oracle's own run only because
AdamW normalizes small gradient differences into full-size updates, so the
comparison is step by step on the GPU's own trajectory: every GPU step starts
from the state the previous GPU step left, and the oracle recomputes that step
from the same state.  Checked per step: the schedule (block, epoch, sample, step
count), the loss and the gradient against the oracle at the GPU's parameters on
the oracle's target for that sample (2e-2 relative, the bf16 matrix-core path),
and the AdamW update and moments from the GPU's gradient (1e-4).  Per block: the
starting parameters, the inputs (the samples for block 0, then the previous
block's quantized outputs against the oracle's, 2e-2), and the final outputs.
Cases: a 2-block stack of 7B-shaped W4A4 blocks with s_a (multi-head), and of
grouped-query W2A16 blocks with 128-channel LWC groups; 2 samples, 2 epochs.
"""
import numpy as np
import pytest
import torch

import post_quantization_amd as omq
from post_quantization_amd import driver
from oracle import block as ob
from oracle import driver as od
from oracle import optim
import synth
from gpu_util import DEV, dev, host, log, rel

pytestmark = pytest.mark.gpu

F32 = np.float32
TOL = 2e-2

CASES = {
    "mha_w4a4": synth.reduced(synth.BLOCK_CFG4, T=256, d=512, n_q=4, n_kv=4, F=1376, n_out=5),
    "gqa_w2a16g128": synth.reduced(synth.BLOCK_CFG4_W2G128, T=192, d=512, n_q=4, n_kv=2,
                                   F=1408, n_out=5),
}


def desc_of(c):
    return omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                         wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group,
                         eps=c.eps, rope_theta=c.rope_theta, lr_lwc=c.lr_lwc, lr_let=c.lr_let)


@pytest.mark.parametrize("kind", list(CASES))
def test_driver_stepwise(kind):
    c = CASES[kind]
    n_blocks, n_samples, epochs = 2, 2, 2
    log("driver", kind, c)
    blocks, xs = synth.stack_inputs(c, n_blocks, n_samples)
    d = desc_of(c)
    W = [[dev(Wd["W_" + n], torch.bfloat16) for n in synth.WEIGHT_NAMES] for Wd in blocks]
    steps, inputs = [], {}

    def on_step(s):
        steps.append((s.block, s.epoch, s.sample, s.step, host(s.theta).copy(),
                      host(s.dtheta).copy(), host(s.adam_m).copy(), host(s.adam_v).copy(),
                      float(host(s.loss)[0])))

    res = driver.calibrate(d, W, dev(xs, torch.bfloat16), epochs, on_step=on_step,
                           on_block=lambda b, x, th: inputs.setdefault(b, host(x).copy()))
    torch.cuda.synchronize()
    want = [(b, e, i, e * n_samples + i + 1) for b in range(n_blocks) for e in range(epochs)
            for i in range(n_samples)]
    assert [s[:4] for s in steps] == want

    shapes = synth.block_weight_shapes(c)
    init = ob.pack(c, shapes, ob.init_theta(c, shapes))
    offs, n_lwc, total = omq.block_theta_layout(d)
    assert init.size == total
    assert np.array_equal(inputs[0], xs)
    for b in range(n_blocks):
        Wd = blocks[b]
        xb = [inputs[b][i].astype(np.float64) for i in range(n_samples)]
        if b > 0:
            # this block's inputs: the previous block's quantized outputs
            prev = od.next_inputs(c, blocks[b - 1], host(res.thetas[b - 1]),
                                  [inputs[b - 1][i].astype(np.float64) for i in range(n_samples)])
            for i in range(n_samples):
                e = rel(xb[i], prev[i])
                log("block", b, "input", i, "rel %.2e" % e)
                assert e < TOL
        ys = od.targets(c, Wd, xb)
        pre = (init, np.zeros(total, F32), np.zeros(total, F32))
        for (bb, e, i, t, th, g, m, v, loss) in [s for s in steps if s[0] == b]:
            vec_o, m_o, v_o, loss_o, g_o = od.step(c, shapes, Wd, xb[i], ys[i], *pre, t)
            eg = rel(g, g_o)
            log("block", b, "epoch", e, "sample", i, "loss %.4e / %.4e" % (loss, loss_o),
                "grad rel %.2e" % eg)
            assert abs(loss - loss_o) <= TOL * loss_o
            assert eg < TOL
            # AdamW from the step's own gradient, per parameter group
            exp = [optim.adamw(pre[0][sl], g[sl], pre[1][sl], pre[2][sl], t, lr)
                   for sl, lr in ((slice(0, n_lwc), c.lr_lwc), (slice(n_lwc, total), c.lr_let))]
            th_e = np.concatenate([x[0] for x in exp])
            assert rel(th - pre[0], th_e - pre[0]) < 1e-4
            assert rel(m, np.concatenate([x[1] for x in exp])) < 1e-4
            assert rel(v, np.concatenate([x[2] for x in exp])) < 1e-4
            pre = (th, m, v)
        assert np.array_equal(host(res.thetas[b]), pre[0])
    out = od.next_inputs(c, blocks[-1], host(res.thetas[-1]),
                         [inputs[n_blocks - 1][i].astype(np.float64) for i in range(n_samples)])
    got = host(res.outputs)
    for i in range(n_samples):
        assert rel(got[i], out[i]) < TOL


def test_driver_resume_matches():
    """Given the first block's calibrated parameters (resume), the driver advances
    the inputs through it and calibrates the rest as the full run did: bit for bit
    up to the second block's first step (the forward passes are deterministic), then
    up to the order of the floating-point atomic additions that scatter the
    clipping range's gradient into the LET-scale gradient."""
    c = CASES["gqa_w2a16g128"]
    blocks, xs = synth.stack_inputs(c, 2, 2)
    d = desc_of(c)
    W = [[dev(Wd["W_" + n], torch.bfloat16) for n in synth.WEIGHT_NAMES] for Wd in blocks]
    x = dev(xs, torch.bfloat16)
    full = driver.calibrate(d, W, x, 1)
    again = driver.calibrate(d, W, x, 1, done=[full.thetas[0]])
    torch.cuda.synchronize()
    assert torch.equal(again.thetas[0], full.thetas[0])
    assert torch.equal(x, dev(xs, torch.bfloat16))
    t0, t1 = host(full.thetas[1]), host(again.thetas[1])
    init = host(driver.init_theta(d, DEV))
    assert rel(t1 - init, t0 - init) < 1e-4
    assert rel(host(again.outputs), host(full.outputs)) < 1e-3
