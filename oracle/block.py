"""Oracle LLaMA-shaped decoder block with OmniQuant's quantizers, its
full-precision target, the MSE objective, and the hand-written backward.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows the paper reading "OmniQuant ..." (onecrewdev.com):
* section "框架": the block-wise objective || F(W, X) - F(Q_w(W), Q_a(X)) || over
  Theta1 = {gamma, beta} and Theta2 = {delta, s, s_a}, weights frozen;
* section "LET": LET on every linear except the second FFN linear (down_proj);
  the attention affinity Softmax(Q K^T) = Softmax((Q / s_a)(s_a * K)^T); Q, K, V
  quantized (low-bit KV cache); the softmax output kept in full precision.

Readings of what the pages leave open:
* the norm of the objective is the mean squared error over tokens x hidden;
* RMSNorm with eps 1e-6 and unit gain; RoPE (rotate-half, theta 10000,
  positions 0..T-1); SiLU gating; no biases (B = 0, so B~ = delta W);
* scaled (1/sqrt(head_dim)) causal attention;
* s_a acts on the post-RoPE Q and K entering Q K^T; Q~, K~ and V are quantized
  per token over all heads' channels; s_a is only learned when activations are
  quantized (without a quantizer Q K^T does not depend on it);
* LET sites: one (s, delta) shared by the q/k/v input, one by the gate/up input,
  one on the o_proj input; with grouped-query attention s_o, delta_o and s_a live
  on the KV channels and are broadcast over the query heads of each group;
* the block's quantized input is the same x as the full-precision target;
* operand precision of the bf16 path (ops.ExactOps): the forward product of
  every layer with both quantizers on takes the exact dequantized operands (the
  method's Y = Q_a(X~) Q_w(W~) + B~); every other product takes bf16 operands.

Parity: pinned by tests/test_oracle_block.py (full-precision block vs torch's
rms_norm / scaled_dot_product_attention / silu; RoPE invariants; LET identity of
the whole block at W16A16; zero LET gradients at W16A16; finite differences of
the frozen-decision surrogate for every parameter group).
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

from . import quant
from .ops import ExactOps

F32 = np.float32
F64 = np.float64

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")


# ---------------------------------------------------------------------------
# smooth pieces (float64)
# ---------------------------------------------------------------------------

def rmsnorm(x, eps, code=True):
    """RMSNorm with unit gain, y = x / sqrt(mean(x^2) + eps), and the scale r.

    code: the output enters a quantizer, so its rounding is fixed like the
    quantizer's (reading R29): r is formed in float64 (eps as the float32 the GPU
    takes) and rounded once to float32, the normalized row is x r rounded once to
    float32 per element.  code=False: everything in float64 (the full-precision
    target, which feeds no quantizer)."""
    x = np.asarray(x, F64)
    if not code:
        r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
        return x * r[:, None], r
    r = (1.0 / np.sqrt(np.mean(x * x, axis=1) + float(F32(eps)))).astype(F32).astype(F64)
    return (x * r[:, None]).astype(F32).astype(F64), r


def rmsnorm_bwd(dy, x, r):
    x = np.asarray(x, F64)
    d = x.shape[1]
    dot = np.sum(dy * x, axis=1)
    return r[:, None] * dy - x * (r ** 3 * dot / d)[:, None]


def rope_tables(T, hd, theta):
    half = hd // 2
    inv = theta ** (-np.arange(half, dtype=F64) * 2.0 / hd)
    ang = np.arange(T, dtype=F64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, n_heads, hd, cos, sin):
    """Rotate-half RoPE on every head of x [T, n_heads*hd]."""
    T = x.shape[0]
    v = np.asarray(x, F64).reshape(T, n_heads, hd)
    half = hd // 2
    a, b = v[..., :half], v[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1).reshape(T, n_heads * hd)


def rope_bwd(g, n_heads, hd, cos, sin):
    T = g.shape[0]
    v = np.asarray(g, F64).reshape(T, n_heads, hd)
    half = hd // 2
    a, b = v[..., :half], v[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1).reshape(T, n_heads * hd)


def silu(x):
    return x / (1.0 + np.exp(-x))


def attention(Q, K, V, n_q, n_kv, hd, cast=None):
    """Causal scaled attention, float64 softmax.  Q [T, n_q*hd], K/V [T, n_kv*hd].

    cast: how the probabilities enter the P V product (the bf16 path feeds them to
    the matrix cores in bf16); the softmax itself is never quantized."""
    T = Q.shape[0]
    grp = n_q // n_kv
    c = 1.0 / np.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    O = np.zeros((T, n_q * hd))
    P = []
    for h in range(n_q):
        g = h // grp
        q = Q[:, h * hd:(h + 1) * hd]
        k = K[:, g * hd:(g + 1) * hd]
        v = V[:, g * hd:(g + 1) * hd]
        S = (q @ k.T) * c
        S[mask] = -np.inf
        S = S - S.max(axis=1, keepdims=True)
        E = np.exp(S)
        Ph = E / E.sum(axis=1, keepdims=True)
        Pop = Ph if cast is None else cast(Ph)
        O[:, h * hd:(h + 1) * hd] = Pop @ v
        P.append((Ph, Pop))
    return O, P


def attention_bwd(dO, Q, K, V, P, n_q, n_kv, hd, cast=None):
    """Backward of attention(); cast: how dO and dS enter their matrix products (the
    bf16 path feeds them to the matrix cores in bf16).  The softmax term
    rowsum(dP P) is formed from the uncast dO as rowsum(dO O)."""
    cast = (lambda a: a) if cast is None else cast
    T = Q.shape[0]
    grp = n_q // n_kv
    c = 1.0 / np.sqrt(hd)
    dQ = np.zeros_like(Q, dtype=F64)
    dK = np.zeros_like(K, dtype=F64)
    dV = np.zeros_like(V, dtype=F64)
    for h in range(n_q):
        g = h // grp
        sl_q = slice(h * hd, (h + 1) * hd)
        sl_k = slice(g * hd, (g + 1) * hd)
        do = dO[:, sl_q]
        doc = cast(do)
        Ph, Pop = P[h]
        dV[:, sl_k] += Pop.T @ doc
        dP = doc @ V[:, sl_k].T
        # rowsum(dP P) written as rowsum(dO O) with O = P V, the product the forward
        # formed (its P operand the cast one)
        Dr = np.sum((do @ V[:, sl_k].T) * Pop, axis=1, keepdims=True)
        dS = cast(c * (Ph * (dP - Dr)))
        dQ[:, sl_q] = dS @ K[:, sl_k]
        dK[:, sl_k] += dS.T @ Q[:, sl_q]
    return dQ, dK, dV


def kv_broadcast(vec, n_q, n_kv, hd):
    """A per-KV-channel vector [n_kv*hd] spread over the query heads [n_q*hd]."""
    grp = n_q // n_kv
    v = np.asarray(vec).reshape(n_kv, 1, hd)
    return np.broadcast_to(v, (n_kv, grp, hd)).reshape(n_q * hd)


def kv_reduce(vec, n_q, n_kv, hd):
    """Adjoint of kv_broadcast: sum the query heads of each group."""
    grp = n_q // n_kv
    return np.asarray(vec, F64).reshape(n_kv, grp, hd).sum(axis=1).reshape(n_kv * hd)


# ---------------------------------------------------------------------------
# parameters
# ---------------------------------------------------------------------------

def linears(c):
    return ("gate", "up", "down") if c.ffn_only else LINEARS


def let_sites(c):
    return ("ffn",) if c.ffn_only else ("qkv", "o", "ffn")


def uses_sa(c):
    return (not c.ffn_only) and c.abits < 16


def lwc_rows(c, shape):
    """Quantizer rows of one weight [C_out, C_in]: one per output channel, or one
    per group of c.group input channels (group-wise LWC)."""
    C_out, C_in = shape
    if c.group:
        assert C_in % c.group == 0, (C_in, c.group)
        return C_out * (C_in // c.group)
    return C_out


def theta_layout(c, shapes):
    """Packed order: per linear a_gamma[rows], a_beta[rows] (rows = C_out, or
    C_out * C_in / group output-channel major for group-wise LWC); per LET site
    s[C], delta[C]; then s_a[C_k].  Returns [(name, size)]."""
    out = []
    for n in linears(c):
        out.append(("a_gamma_" + n, lwc_rows(c, shapes[n])))
        out.append(("a_beta_" + n, lwc_rows(c, shapes[n])))
    kvd = c.n_kv * c.head_dim
    site_dim = {"qkv": c.d, "o": kvd, "ffn": c.d}
    for s in let_sites(c):
        out.append(("s_" + s, site_dim[s]))
        out.append(("delta_" + s, site_dim[s]))
    if uses_sa(c):
        out.append(("s_a", kvd))
    return out


def init_theta(c, shapes, a0=4.0):
    th = {}
    for name, n in theta_layout(c, shapes):
        if name.startswith("a_"):
            th[name] = np.full(n, a0, F32)
        elif name.startswith("delta_"):
            th[name] = np.zeros(n, F32)
        else:
            th[name] = np.ones(n, F32)
    return th


def pack(c, shapes, th):
    return np.concatenate([np.asarray(th[n], F32).reshape(-1) for n, _ in theta_layout(c, shapes)])


def unpack(c, shapes, flat):
    out, o = {}, 0
    for n, k in theta_layout(c, shapes):
        out[n] = np.asarray(flat[o:o + k], F32)
        o += k
    return out


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def _qlin(ops, S, name, Xop, W, th, c, s=None, delta=None, Xfw=None):
    """One quantized linear on an already-quantized operand Xop (the backward's
    operand); Xfw, when given, is the exact quantized input the forward product
    takes instead, with the exact quantized weight."""
    gamma = ops.sigmoid(th["a_gamma_" + name])
    beta = ops.sigmoid(th["a_beta_" + name])
    Wt = ops.let_weight(W, s) if s is not None else ops.to_code(W)
    if c.wbits >= 16:               # weight quantizer off
        wst = None
        Wop = ops.operand(Wt)
    else:
        # one quantizer row per output channel, or per group of input channels
        rows = lwc_rows(c, Wt.shape)
        wst = ops.quant(np.reshape(Wt, (rows, -1)), gamma, beta, c.wbits, "w_" + name)
        Wop = ops.operand(np.reshape(wst.xhat, Wt.shape))
    if Xfw is not None and wst is not None:
        Y = np.asarray(Xfw, F64) @ np.reshape(wst.xhat, Wt.shape).astype(F64).T
    else:
        Y = Xop @ Wop.T
    if delta is not None:
        Y = Y + quant.bias_fold(W, None, delta)[None, :]
    S[name] = SimpleNamespace(gamma=gamma, beta=beta, wst=wst, Wop=Wop, W=W, s=s, Y=Y)
    return Y


def forward(c, x, Wd, th, ops=None):
    """Quantized block forward.  x [T, d] (bf16 values), Wd: dict of weights."""
    if ops is None:
        ops = ExactOps(bf16=True)
    S = SimpleNamespace(c=c, ops=ops, th=th)
    S.lin = {}
    # weight-activation quantized products on their exact operands (method level)
    ep = getattr(ops, "exact_product", None)
    exact = ep is not None and ep(c.wbits, c.abits)

    def fw(Xh):
        return Xh if exact else None
    x64 = np.asarray(x, F64)
    hd, n_q, n_kv = c.head_dim, c.n_q, c.n_kv
    sv = {}
    if not c.ffn_only:
        rr = getattr(ops, "rms_rounding", False)
        xn, r1 = rmsnorm(x64, c.eps, code=rr)
        s_qkv, d_qkv = th["s_qkv"], th["delta_qkv"]
        Xt_qkv = ops.let_act(xn, s_qkv, d_qkv)
        a_qkv, Xh = ops.act(Xt_qkv, c.abits, "a_qkv")
        Xop_qkv = ops.operand(Xh)
        Yq = _qlin(ops, sv, "q", Xop_qkv, Wd["W_q"], th, c, s_qkv, d_qkv, fw(Xh))
        Yk = _qlin(ops, sv, "k", Xop_qkv, Wd["W_k"], th, c, s_qkv, d_qkv, fw(Xh))
        Yv = _qlin(ops, sv, "v", Xop_qkv, Wd["W_v"], th, c, s_qkv, d_qkv, fw(Xh))
        cos, sin = rope_tables(c.T, hd, c.rope_theta)
        Qr = rope(Yq, n_q, hd, cos, sin)
        Kr = rope(Yk, n_kv, hd, cos, sin)
        if uses_sa(c):
            sa_k = th["s_a"]
            sa_q = kv_broadcast(sa_k, n_q, n_kv, hd)
            Qt = ops.div(Qr, sa_q)
            Kt = ops.mul(Kr, sa_k)
        else:
            sa_k = sa_q = None
            Qt, Kt = Qr, Kr
        aQ, Qh = ops.act(Qt, c.abits, "a_q")
        aK, Kh = ops.act(Kt, c.abits, "a_k")
        aV, Vh = ops.act(Yv, c.abits, "a_v")
        Qo, Ko, Vo = ops.operand(Qh), ops.operand(Kh), ops.operand(Vh)
        O, P = attention(Qo, Ko, Vo, n_q, n_kv, hd, cast=getattr(ops, "prob", ops.operand))
        s_o = kv_broadcast(th["s_o"], n_q, n_kv, hd)
        d_o = kv_broadcast(th["delta_o"], n_q, n_kv, hd)
        Xt_o = ops.let_act(O, s_o, d_o)
        a_o, Xh_o = ops.act(Xt_o, c.abits, "a_o")
        Xop_o = ops.operand(Xh_o)
        h1 = x64 + _qlin(ops, sv, "o", Xop_o, Wd["W_o"], th, c, s_o, d_o, fw(Xh_o))
        xn2, r2 = rmsnorm(h1, c.eps, code=rr)
        S.__dict__.update(xn=xn, r1=r1, Xt_qkv=Xt_qkv, a_qkv=a_qkv, Xop_qkv=Xop_qkv,
                          cos=cos, sin=sin, Qr=Qr, Kr=Kr, Qt=Qt, Kt=Kt, Yv=Yv, sa_q=sa_q,
                          sa_k=sa_k, aQ=aQ, aK=aK, aV=aV, Qo=Qo, Ko=Ko, Vo=Vo, O=O, P=P,
                          s_o=s_o, d_o=d_o, Xt_o=Xt_o, a_o=a_o, Xop_o=Xop_o, h1=h1, r2=r2)
    else:
        h1 = None
        xn2 = x64
    s_f, d_f = th["s_ffn"], th["delta_ffn"]
    Xt_f = ops.let_act(xn2, s_f, d_f)
    a_f, Xh_f = ops.act(Xt_f, c.abits, "a_ffn")
    Xop_f = ops.operand(Xh_f)
    G = _qlin(ops, sv, "gate", Xop_f, Wd["W_gate"], th, c, s_f, d_f, fw(Xh_f))
    U = _qlin(ops, sv, "up", Xop_f, Wd["W_up"], th, c, s_f, d_f, fw(Xh_f))
    A = silu(G) * U
    a_d, Xh_d = ops.act(A, c.abits, "a_down")
    Xop_d = ops.operand(Xh_d)
    D = _qlin(ops, sv, "down", Xop_d, Wd["W_down"], th, c, Xfw=fw(Xh_d))
    y = D if c.ffn_only else h1 + D
    S.__dict__.update(xn2=xn2, Xt_f=Xt_f, a_f=a_f, Xop_f=Xop_f, G=G, U=U, A=A, a_d=a_d,
                      Xop_d=Xop_d, y=y)
    S.lin = sv
    return y, S


def reference(c, x, Wd):
    """Full-precision block output y* (raw weights, no quantizers), float64."""
    x64 = np.asarray(x, F64)
    W = {k: np.asarray(v, F64) for k, v in Wd.items()}
    hd, n_q, n_kv = c.head_dim, c.n_q, c.n_kv
    if c.ffn_only:
        xn2 = x64
        h1 = None
    else:
        xn, _ = rmsnorm(x64, c.eps, code=False)
        cos, sin = rope_tables(c.T, hd, c.rope_theta)
        Q = rope(xn @ W["W_q"].T, n_q, hd, cos, sin)
        K = rope(xn @ W["W_k"].T, n_kv, hd, cos, sin)
        V = xn @ W["W_v"].T
        O, _ = attention(Q, K, V, n_q, n_kv, hd)
        h1 = x64 + O @ W["W_o"].T
        xn2, _ = rmsnorm(h1, c.eps, code=False)
    A = silu(xn2 @ W["W_gate"].T) * (xn2 @ W["W_up"].T)
    D = A @ W["W_down"].T
    return D if c.ffn_only else h1 + D


def mse(y, ystar):
    diff = np.asarray(y, F64) - np.asarray(ystar, F64)
    return float(np.mean(diff * diff)), 2.0 * diff / diff.size


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _qlin_bwd(S, name, gY, Xop, g, gs=None):
    """Backward of one quantized linear: returns dL/dXop; fills the LWC logit
    grads and accumulates the weight-side s grad into gs."""
    L = S.lin[name]
    gYo = S.ops.grad_operand(gY) if hasattr(S.ops, "grad_operand") else gY
    gXop = gYo @ L.Wop
    gWop = gYo.T @ Xop
    if L.wst is None:
        rows = lwc_rows(S.c, gWop.shape)
        gWt, g_gamma, g_beta = gWop, np.zeros(rows), np.zeros(rows)
    else:
        gWt, g_gamma, g_beta = quant.quantize_rows_bwd(np.reshape(gWop, (L.wst.h.size, -1)),
                                                       L.wst)
        gWt = np.reshape(gWt, gWop.shape)
    ga, gb = L.gamma.astype(F64), L.beta.astype(F64)
    g["a_gamma_" + name] = g_gamma * ga * (1.0 - ga)
    g["a_beta_" + name] = g_beta * gb * (1.0 - gb)
    if gs is not None:
        gs += np.sum(gWt * np.asarray(L.W, F64), axis=0)
    return gXop


def _let_act_bwd(gXt, Xt, s):
    """X~ = (X - delta) / s: returns (gX, g_s, g_delta)."""
    s = np.asarray(s, F64)
    Xt = np.asarray(Xt, F64)
    g_s = np.sum(gXt * (-Xt / s[None, :]), axis=0)
    g_d = np.sum(gXt, axis=0) * (-1.0 / s)
    return gXt / s[None, :], g_s, g_d


def backward(S, dy):
    """Gradients of the objective w.r.t. every learnable parameter (dict)."""
    c = S.c
    hd, n_q, n_kv = c.head_dim, c.n_q, c.n_kv
    dy = np.asarray(dy, F64)
    g = {}
    # FFN second linear (no LET)
    gXop_d = _qlin_bwd(S, "down", dy, S.Xop_d, g)
    gA = quant.act_quant_bwd(gXop_d, S.a_d)
    sg = 1.0 / (1.0 + np.exp(-S.G))
    gG = gA * S.U * sg * (1.0 + S.G * (1.0 - sg))
    gU = gA * S.G * sg
    # gate / up with the shared ffn LET site
    gs_f = np.zeros(S.Xt_f.shape[1])
    gXop_f = _qlin_bwd(S, "gate", gG, S.Xop_f, g, gs_f) + _qlin_bwd(S, "up", gU, S.Xop_f, g, gs_f)
    gXt_f = quant.act_quant_bwd(gXop_f, S.a_f)
    gxn2, gs2, gd_f = _let_act_bwd(gXt_f, S.Xt_f, S.th["s_ffn"])
    W_g = np.asarray(S.lin["gate"].W, F64)
    W_u = np.asarray(S.lin["up"].W, F64)
    g["s_ffn"] = gs_f + gs2
    g["delta_ffn"] = gd_f + W_g.T @ gG.sum(axis=0) + W_u.T @ gU.sum(axis=0)
    if c.ffn_only:
        return g
    dh1 = dy + rmsnorm_bwd(gxn2, S.h1, S.r2)
    # o_proj with its LET site
    gs_o = np.zeros(n_q * hd)
    gXop_o = _qlin_bwd(S, "o", dh1, S.Xop_o, g, gs_o)
    gXt_o = quant.act_quant_bwd(gXop_o, S.a_o)
    gO, gs_o2, gd_o = _let_act_bwd(gXt_o, S.Xt_o, S.s_o)
    gd_o = gd_o + np.asarray(S.lin["o"].W, F64).T @ dh1.sum(axis=0)
    g["s_o"] = kv_reduce(gs_o + gs_o2, n_q, n_kv, hd)
    g["delta_o"] = kv_reduce(gd_o, n_q, n_kv, hd)
    # attention
    gQo, gKo, gVo = attention_bwd(gO, S.Qo, S.Ko, S.Vo, S.P, n_q, n_kv, hd,
                                  cast=getattr(S.ops, "grad_operand", None))
    gQt = quant.act_quant_bwd(gQo, S.aQ)
    gKt = quant.act_quant_bwd(gKo, S.aK)
    gYv = quant.act_quant_bwd(gVo, S.aV)
    if uses_sa(c):
        sa_q = np.asarray(S.sa_q, F64)
        sa_k = np.asarray(S.sa_k, F64)
        Qt = np.asarray(S.Qt, F64)
        gsa_q = np.sum(gQt * (-Qt / sa_q[None, :]), axis=0)
        gsa_k = np.sum(gKt * np.asarray(S.Kr, F64), axis=0)
        g["s_a"] = kv_reduce(gsa_q, n_q, n_kv, hd) + gsa_k
        gQr = gQt / sa_q[None, :]
        gKr = gKt * sa_k[None, :]
    else:
        gQr, gKr = gQt, gKt
    gYq = rope_bwd(gQr, n_q, hd, S.cos, S.sin)
    gYk = rope_bwd(gKr, n_kv, hd, S.cos, S.sin)
    gs_qkv = np.zeros(c.d)
    gXop = (_qlin_bwd(S, "q", gYq, S.Xop_qkv, g, gs_qkv)
            + _qlin_bwd(S, "k", gYk, S.Xop_qkv, g, gs_qkv)
            + _qlin_bwd(S, "v", gYv, S.Xop_qkv, g, gs_qkv))
    gXt = quant.act_quant_bwd(gXop, S.a_qkv)
    _, gs3, gd = _let_act_bwd(gXt, S.Xt_qkv, S.th["s_qkv"])
    g["s_qkv"] = gs_qkv + gs3
    g["delta_qkv"] = gd + sum(np.asarray(S.lin[n].W, F64).T @ gy.sum(axis=0)
                              for n, gy in (("q", gYq), ("k", gYk), ("v", gYv)))
    return g


def calib_step(c, x, Wd, ystar, th, ops=None):
    """One forward + MSE + backward; returns (loss, grads, y, saved)."""
    y, S = forward(c, x, Wd, th, ops)
    loss, dy = mse(y, ystar)
    return loss, backward(S, dy), y, S
