"""Pins of the oracle block (CPU only).

* The full-precision block equals one assembled from torch's library routines
  (rms_norm, scaled_dot_product_attention with a causal mask, silu) with RoPE
  applied as a complex rotation (an independent formulation of rotate-half).
* RoPE invariants: it preserves norms and q.k depends only on relative position.
* Attention and RMSNorm backward equal torch autograd (float64).
* LET identity ("strictly equivalent" transform): with quantizers off the
  quantized block with random s > 0, delta and the fp32 LET equals the
  full-precision block; softmax(Q~ K~^T) = softmax(Q K^T) for any s_a > 0.
* With quantizers off the objective does not depend on s, delta, s_a or the
  clipping logits, so their gradients vanish (gamma/beta exactly).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import block as ob
from oracle.ops import ExactOps
import synth

F32 = np.float32
F64 = np.float64


def _cfg(**kw):
    base = dict(cfg=4, T=24, d=32, n_q=4, n_kv=2, F=40, wbits=16, abits=16, head_dim=8,
                n_out=3, out_lo=5.0, out_hi=20.0)
    base.update(kw)
    return synth.BlockCfg(**base)


def _torch_block(c, x, Wd):
    t = lambda a: torch.from_numpy(np.asarray(a, F64))
    x = t(x)
    W = {k: t(v) for k, v in Wd.items()}
    T, hd = c.T, c.head_dim

    def rope_c(v, nh):
        v = v.reshape(T, nh, 2, hd // 2).permute(0, 1, 3, 2).contiguous()
        z = torch.view_as_complex(v)
        inv = c.rope_theta ** (-torch.arange(hd // 2, dtype=torch.float64) * 2 / hd)
        ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
        z = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
        r = torch.view_as_real(z).permute(0, 1, 3, 2).reshape(T, nh * hd)
        return r

    xn = Fn.rms_norm(x, (c.d,), eps=c.eps)
    q = rope_c(xn @ W["W_q"].T, c.n_q).reshape(T, c.n_q, hd).transpose(0, 1)
    k = rope_c(xn @ W["W_k"].T, c.n_kv).reshape(T, c.n_kv, hd).transpose(0, 1)
    v = (xn @ W["W_v"].T).reshape(T, c.n_kv, hd).transpose(0, 1)
    rep = c.n_q // c.n_kv
    k = k.repeat_interleave(rep, 0)
    v = v.repeat_interleave(rep, 0)
    o = Fn.scaled_dot_product_attention(q, k, v, is_causal=True)
    o = o.transpose(0, 1).reshape(T, c.n_q * hd)
    h1 = x + o @ W["W_o"].T
    xn2 = Fn.rms_norm(h1, (c.d,), eps=c.eps)
    a = Fn.silu(xn2 @ W["W_gate"].T) * (xn2 @ W["W_up"].T)
    return (h1 + a @ W["W_down"].T).numpy()


@pytest.mark.parametrize("n_q,n_kv", [(4, 4), (4, 2), (4, 1)])
def test_reference_block_vs_torch(n_q, n_kv):
    c = _cfg(n_q=n_q, n_kv=n_kv)
    inp = synth.block_inputs(c)
    Wd = {k: v * 20 for k, v in inp.items() if k.startswith("W_")}
    y = ob.reference(c, inp["x"], Wd)
    yt = _torch_block(c, inp["x"], Wd)
    assert np.linalg.norm(y - yt) / np.linalg.norm(yt) < 1e-12


def test_rope_invariants():
    rng = np.random.default_rng(0)
    T, hd = 40, 16
    cos, sin = ob.rope_tables(T, hd, 10000.0)
    q = rng.standard_normal((T, hd))
    k = rng.standard_normal((T, hd))
    rq = ob.rope(q, 1, hd, cos, sin)
    assert np.allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q, axis=1))
    assert np.allclose(rq[0], q[0])
    # same vectors at every position: rotated dot product depends on i - j only
    qq = np.repeat(q[:1], T, 0)
    kk = np.repeat(k[:1], T, 0)
    dots = ob.rope(qq, 1, hd, cos, sin) @ ob.rope(kk, 1, hd, cos, sin).T
    for off in (0, 3, 11):
        dg = np.diagonal(dots, offset=off)
        assert np.allclose(dg, dg[0])
    # backward is the adjoint (transpose) of the forward rotation
    g = rng.standard_normal((T, hd))
    assert np.isclose(np.sum(g * rq), np.sum(ob.rope_bwd(g, 1, hd, cos, sin) * q))


def test_attention_and_rmsnorm_bwd_vs_autograd():
    rng = np.random.default_rng(1)
    T, hd, n_q, n_kv = 12, 8, 4, 2
    Q = rng.standard_normal((T, n_q * hd))
    K = rng.standard_normal((T, n_kv * hd))
    V = rng.standard_normal((T, n_kv * hd))
    dO = rng.standard_normal((T, n_q * hd))
    O, P = ob.attention(Q, K, V, n_q, n_kv, hd)
    dQ, dK, dV = ob.attention_bwd(dO, Q, K, V, P, n_q, n_kv, hd)
    tQ, tK, tV = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    q = tQ.reshape(T, n_q, hd).transpose(0, 1)
    k = tK.reshape(T, n_kv, hd).transpose(0, 1).repeat_interleave(n_q // n_kv, 0)
    v = tV.reshape(T, n_kv, hd).transpose(0, 1).repeat_interleave(n_q // n_kv, 0)
    o = Fn.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(T, -1)
    assert np.allclose(o.detach().numpy(), O, atol=1e-12)
    o.backward(torch.tensor(dO))
    for a, b in ((dQ, tQ), (dK, tK), (dV, tV)):
        assert np.allclose(a, b.grad.numpy(), atol=1e-10)
    x = rng.standard_normal((T, 16)) * 3
    dy = rng.standard_normal((T, 16))
    y, r = ob.rmsnorm(x, 1e-6, code=False)
    tx = torch.tensor(x, requires_grad=True)
    Fn.rms_norm(tx, (16,), eps=1e-6).backward(torch.tensor(dy))
    assert np.allclose(ob.rmsnorm_bwd(dy, x, r), tx.grad.numpy(), atol=1e-10)


def _random_theta(c, shapes, rng):
    th = ob.init_theta(c, shapes)
    for k in th:
        if k.startswith("s"):
            th[k] = rng.uniform(0.4, 2.5, th[k].size).astype(F32)
        elif k.startswith("delta"):
            th[k] = (rng.standard_normal(th[k].size) * 0.5).astype(F32)
        else:
            th[k] = rng.uniform(0.0, 5.0, th[k].size).astype(F32)
    return th


@pytest.mark.parametrize("ffn_only", [False, True])
def test_let_identity_whole_block(ffn_only):
    c = _cfg(ffn_only=ffn_only)
    inp = synth.block_inputs(c)
    Wd = {k: v for k, v in inp.items() if k.startswith("W_")}
    shapes = synth.block_weight_shapes(c)
    th = _random_theta(c, shapes, np.random.default_rng(2))
    y, _ = ob.forward(c, inp["x"], Wd, th, ExactOps(bf16=False))
    ys = ob.reference(c, inp["x"], Wd)
    assert np.linalg.norm(y - ys) / np.linalg.norm(ys) < 1e-5


def test_let_identity_attention_affinity():
    rng = np.random.default_rng(4)
    T, hd = 10, 8
    Q = rng.standard_normal((T, hd)).astype(F32)
    K = rng.standard_normal((T, hd)).astype(F32)
    V = rng.standard_normal((T, hd))
    sa = rng.uniform(0.3, 3.0, hd).astype(F32)
    ops = ExactOps(bf16=False)
    O1, _ = ob.attention(Q.astype(F64), K.astype(F64), V, 1, 1, hd)
    O2, _ = ob.attention(ops.div(Q, sa).astype(F64), ops.mul(K, sa).astype(F64), V, 1, 1, hd)
    assert np.linalg.norm(O1 - O2) / np.linalg.norm(O1) < 1e-6


def test_let_gradients_vanish_without_quantizers():
    c = _cfg()
    inp = synth.block_inputs(c)
    Wd = {k: v * 10 for k, v in inp.items() if k.startswith("W_")}
    shapes = synth.block_weight_shapes(c)
    rng = np.random.default_rng(3)
    th = _random_theta(c, shapes, rng)
    target = ob.reference(c, inp["x"], Wd) + rng.standard_normal((c.T, c.d))
    loss, g, y, S = ob.calib_step(c, inp["x"], Wd, target, th, ExactOps(bf16=False))
    assert loss > 0.1
    for n, v in g.items():
        if n.startswith("a_"):
            assert np.all(v == 0), n
        else:
            # LET parameters: the act-side and weight-side terms cancel
            assert np.abs(v).max() < 1e-5 * max(1.0, loss), (n, np.abs(v).max())


@pytest.mark.parametrize("kw", [dict(wbits=4, abits=4, F=96), dict(wbits=8, abits=8, F=96),
                                dict(wbits=4, abits=4, F=40),
                                dict(wbits=3, abits=6, F=96, group=32)],
                         ids=["w4a4", "w8a8", "w4a4_width40", "w3a6_g32"])
def test_forward_quantized_products_are_exact(kw):
    """The quantized layer is Y = Q_a(X~) Q_w(W~) + B~ (section "LET") with each
    quantized operand (q - z) h per quantizer row (section "LWC").  With both
    quantizers on, the oracle's forward products equal that definition written on
    the integer codes (plus the folded bias), whatever the bit widths, the input
    widths or the LWC grouping; the backward keeps the bf16 path's operands."""
    c = _cfg(T=32, d=64, n_q=2, n_kv=2, head_dim=32, **kw)
    ops = ExactOps(bf16=True)
    assert ops.exact_product(c.wbits, c.abits)
    assert not ops.exact_product(16, c.abits) and not ops.exact_product(c.wbits, 16)
    inp = synth.block_inputs(c)
    Wd = {k: v for k, v in inp.items() if k.startswith("W_")}
    shapes = synth.block_weight_shapes(c)
    th = _random_theta(c, shapes, np.random.default_rng(5))
    _, S = ob.forward(c, inp["x"], Wd, th, ops)
    from oracle import quant
    for name, act in (("q", "a_qkv"), ("v", "a_qkv"), ("o", "a_o"), ("up", "a_ffn"),
                      ("down", "a_down")):
        L = S.lin[name]
        a = ops.states[act]
        C_out, C_in = L.Wop.shape
        if c.group:
            # integer codes of each (row, group) with its own step and zero point
            g = C_in // c.group
            qw = (L.wst.codes.reshape(C_out, g, c.group).astype(np.int64)
                  - L.wst.z.reshape(C_out, g, 1).astype(np.int64))
            wdq = (qw * L.wst.h.reshape(C_out, g, 1).astype(F64)).reshape(C_out, C_in)
            xdq = (a.codes.astype(np.int64) - a.z[:, None].astype(np.int64)) * \
                a.h[:, None].astype(F64)
            want = xdq @ wdq.T
        else:
            want = quant.code_product(a.codes, a.h, a.z, L.wst.codes, L.wst.h, L.wst.z)
        site = {"q": "qkv", "v": "qkv", "o": "o", "up": "ffn"}.get(name)
        if site is not None:
            delta = th["delta_" + site] if site != "o" else ob.kv_broadcast(
                th["delta_o"], c.n_q, c.n_kv, c.head_dim)
            want = want + quant.bias_fold(L.W, None, delta)[None, :]
        assert np.allclose(L.Y, want, rtol=1e-6, atol=1e-6 * np.abs(want).max()), name
        # the backward's operand is the bf16 rounding of the same weight
        assert np.array_equal(L.Wop, quant.bf16(L.wst.xhat.reshape(L.Wop.shape)))


class _UnroundedP(ExactOps):
    """The bf16 path with the softmax output fed to P V unrounded."""

    def prob(self, P):
        return np.asarray(P, F64)


# gradient groups whose value moves by more than the bf16 tolerance (2e-2) when the
# bf16 path's operand roundings are removed: the attention side's
_ROUNDING_SENSITIVE = {"a_gamma_q", "a_beta_q", "a_gamma_k", "a_beta_k", "a_gamma_v", "a_beta_v",
                       "a_gamma_o", "a_beta_o", "s_o", "delta_o", "s_a", "delta_qkv",
                       "delta_ffn"}


@pytest.mark.parametrize("theta_kind", ["init", "random"])
def test_rounding_point_sensitivity(theta_kind):
    """How much of the bf16 path's 2e-2 gradient tolerance its rounding points use.

    The oracle's bf16 path (reading R17) rounds every matrix-core operand to bf16
    where the GPU does (weights and activations of the backward products, Q~, K~, V,
    and the softmax output P, reading R20); the exact path rounds nothing.  On the
    7B-shaped W4A4 block at reduced size the loss and the block's update y - x move
    little between the two, the FFN-side gradients (gate/up/down logits, s_ffn) and
    s_qkv by less than the tolerance, but several attention-side groups by more:
    parity at 2e-2 for those (the set _ROUNDING_SENSITIVE) rests on the oracle
    rounding where the kernels round.  P's rounding alone moves s_o by several
    percent."""
    c = synth.reduced(synth.BLOCK_CFG4, T=256, d=512, n_q=4, n_kv=4, F=1376, n_out=5)
    inp = synth.block_inputs(c)
    Wd = {k: v for k, v in inp.items() if k.startswith("W_")}
    shapes = synth.block_weight_shapes(c)
    if theta_kind == "init":
        th = ob.init_theta(c, shapes)
    else:
        rng = np.random.default_rng(7)
        th = ob.init_theta(c, shapes)
        for k in th:
            n = th[k].size
            if k.startswith("a_"):
                th[k] = rng.uniform(2.0, 5.0, n).astype(F32)
            elif k.startswith("delta"):
                th[k] = (rng.standard_normal(n) * 0.05).astype(F32)
            else:
                th[k] = rng.uniform(0.7, 1.4, n).astype(F32)
    x = inp["x"]
    ystar = ob.reference(c, x, Wd)
    lb, gb, yb, _ = ob.calib_step(c, x, Wd, ystar, th, ExactOps(bf16=True))
    le, ge, ye, _ = ob.calib_step(c, x, Wd, ystar, th, ExactOps(bf16=False))
    _, gp, _, _ = ob.calib_step(c, x, Wd, ystar, th, _UnroundedP(bf16=True))

    def rel(a, b):
        a, b = np.asarray(a, F64), np.asarray(b, F64)
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    assert abs(le - lb) < 1e-3 * lb
    assert rel(ye - x, yb - x) < 2.5e-2
    over = set()
    for name, _ in ob.theta_layout(c, shapes):
        gap = rel(ge[name], gb[name])
        print("%-12s exact vs bf16 %.2e, unrounded P vs bf16 %.2e"
              % (name, gap, rel(gp[name], gb[name])))
        assert gap < 1e-1, name
        if gap > 2e-2:
            over.add(name)
    assert over <= _ROUNDING_SENSITIVE, over - _ROUNDING_SENSITIVE
    assert over, "no group exceeds the tolerance: the documented sensitivity is stale"
    # P's bf16 rounding (reading R20) on its own moves the o-site scale by > 1e-2
    assert rel(gp["s_o"], gb["s_o"]) > 1e-2
