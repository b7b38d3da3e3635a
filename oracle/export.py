"""Oracle of the calibrated layer's deployment form: packed integer codes with
their (h, z), the LET transforms folded into neighbouring parameters, and the
weight-only (A16) product computed from the packed codes.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows the paper reading "OmniQuant: ..." (onecrewdev.com):
* section "LET": the equivalent transformation is folded away after calibration
  (s and delta move into the preceding normalization and the layer's bias, and the
  attention-output pair into the value projection, so the deployed model has the
  original structure and no extra operators);
* section "LWC": the deployed weight is the integer code q with its step h and zero
  point z, dequantized as (q - z) h.

Readings (the pages print no layout):
* codes are packed along the input-channel axis into 32-bit words, floor(32 / N)
  codes per word, code j of a word in bits [j N, (j + 1) N), the word's lowest
  column first; a row is ceil(C_in / per_word) words; unused high bits are 0;
* h and z stay float32 (z is integer valued but is not clamped to [0, 2^N - 1]);
* weight-only fold of an input LET site X~ = (X - delta) / s feeding W_hat:
  X~ W_hat^T + B~ = (X / s) W_hat^T + (B~ - W_hat (delta / s)), so the site's 1/s
  becomes the gain of the normalization in front and the layer gets the bias
  B~ - W_hat (delta / s);
* attention-output site (s_o, delta_o per value channel): rows of the softmax sum to
  one, so P (V - delta_o) / s_o = P (V / s_o) - delta_o / s_o exactly; it folds into
  the value projection as h_v / s_o (per output row) and bias (b_v - delta_o) / s_o.

Parity: pinned by tests/test_oracle_export.py (pack / unpack round trip and
hand-built words, the fold identities against the unfolded LET layer, the packed
product against the fake-quant product).
"""
from __future__ import annotations

import numpy as np

from . import quant

F32 = np.float32
F64 = np.float64


def per_word(nbits: int) -> int:
    return 32 // nbits


def pack_codes(codes, nbits: int) -> np.ndarray:
    """uint8 codes [R, C] -> uint32 words [R, ceil(C / per_word)]."""
    codes = np.asarray(codes, dtype=np.uint64)
    R, C = codes.shape
    P = per_word(nbits)
    W = -(-C // P)
    pad = np.zeros((R, W * P), dtype=np.uint64)
    pad[:, :C] = codes
    pad = pad.reshape(R, W, P)
    shifts = (np.arange(P, dtype=np.uint64) * np.uint64(nbits))[None, None, :]
    return np.bitwise_or.reduce(pad << shifts, axis=2).astype(np.uint32)


def unpack_codes(words, nbits: int, C: int) -> np.ndarray:
    """uint32 words [R, W] -> uint8 codes [R, C] (inverse of pack_codes)."""
    words = np.asarray(words, dtype=np.uint64)
    R, W = words.shape
    P = per_word(nbits)
    shifts = (np.arange(P, dtype=np.uint64) * np.uint64(nbits))[None, None, :]
    mask = np.uint64((1 << nbits) - 1)
    out = (words[:, :, None] >> shifts) & mask
    return out.reshape(R, W * P)[:, :C].astype(np.uint8)


def dequant(codes, h, z, group=None) -> np.ndarray:
    """W_hat = (q - z) h in float32, h / z per row or per (row, group)."""
    codes = np.asarray(codes, dtype=F32)
    R, C = codes.shape
    g = C if group is None else group
    h = np.asarray(h, F32).reshape(R, C // g)
    z = np.asarray(z, F32).reshape(R, C // g)
    hz = np.repeat(h, g, axis=1)
    zz = np.repeat(z, g, axis=1)
    return (codes - zz) * hz


def fold_input_site(W_hat, B_tilde, s, delta):
    """Weight-only fold of X~ = (X - delta) / s into (gain, bias): returns
    (gain = 1 / s, bias = B~ - W_hat (delta / s)), float64."""
    s = np.asarray(s, F64)
    d = np.asarray(delta, F64)
    return 1.0 / s, np.asarray(B_tilde, F64) - np.asarray(W_hat, F64) @ (d / s)


def fold_value_site(h_v, b_v, s_o, delta_o):
    """Attention-output site folded into the value projection: per output row of
    W_v, h / s_o and (b_v - delta_o) / s_o (float64)."""
    s_o = np.asarray(s_o, F64)
    return np.asarray(h_v, F64) / s_o, (np.asarray(b_v, F64) - np.asarray(delta_o, F64)) / s_o


def wa16_linear(X, words, h, z, nbits, C, group=None, bias=None):
    """Y = X W_hat^T (+ bias) from packed codes, W_hat rounded to bf16 as the
    matrix-core operand; X as given (bf16 values); float64 product."""
    codes = unpack_codes(words, nbits, C)
    Wop = quant.bf16(dequant(codes, h, z, group))
    Y = np.asarray(X, F64) @ Wop.T
    if bias is not None:
        Y = Y + np.asarray(bias, F64)[None, :]
    return Y


def export_block(c, Wd, th):
    """Deployment form of a calibrated weight-only block (abits = 16, so s_a is not
    learned): per linear the packed codes of Q(W~) with (h, z) and a bias; the
    attention-output pair folded into v; the input sites' 1/s as the gains of the
    norms in front (as the FFN input's scale when the block is the FFN alone).
    Returns {name: float64 / uint32 array}."""
    from . import block as ob
    assert c.abits >= 16
    group = c.group or None
    out = {}

    def lin(name, W, s, delta):
        r = quant.lwc_fakequant(W, th["a_gamma_" + name], th["a_beta_" + name], c.wbits, s,
                                group=group)
        out[name + ".words"] = pack_codes(r.codes, c.wbits)
        out[name + ".h"] = r.h.astype(F64)
        out[name + ".z"] = r.z.astype(F64)
        bias = np.zeros(W.shape[0])
        if delta is not None:
            _, bias = fold_input_site(r.W_hat, quant.bias_fold(W, None, delta), s, delta)
        out[name + ".bias"] = bias

    if not c.ffn_only:
        s, d = th["s_qkv"], th["delta_qkv"]
        for n in ("q", "k", "v"):
            lin(n, Wd["W_" + n], s, d)
        G = out["v.h"].size // Wd["W_v"].shape[0]
        h2, b2 = fold_value_site(out["v.h"].reshape(-1, G), out["v.bias"][:, None],
                                 np.asarray(th["s_o"], F64)[:, None],
                                 np.asarray(th["delta_o"], F64)[:, None])
        out["v.h"], out["v.bias"] = h2.reshape(-1), b2[:, 0]
        out["attn_norm.gain"] = 1.0 / np.asarray(s, F64)
        s_o = ob.kv_broadcast(th["s_o"], c.n_q, c.n_kv, c.head_dim)
        d_o = ob.kv_broadcast(th["delta_o"], c.n_q, c.n_kv, c.head_dim)
        lin("o", Wd["W_o"], s_o, None)
        out["o.bias"] = quant.bias_fold(Wd["W_o"], None, d_o)
    s, d = th["s_ffn"], th["delta_ffn"]
    lin("gate", Wd["W_gate"], s, d)
    lin("up", Wd["W_up"], s, d)
    lin("down", Wd["W_down"], None, None)
    out["ffn_in.gain"] = 1.0 / np.asarray(s, F64)
    return out


def deployed_forward(c, x, exp, cast=None):
    """The exported block run with its original operators only: norm (times the
    folded gain), linears from packed codes plus bias, RoPE, causal attention,
    SiLU gate, residuals.  cast: how a weight enters its product (None: exact)."""
    from . import block as ob
    cast = cast or (lambda a: np.asarray(a, F64))
    group = c.group or None

    def dlin(name, X, N, K):
        W = dequant(unpack_codes(exp[name + ".words"], c.wbits, K), exp[name + ".h"],
                    exp[name + ".z"], group)
        return np.asarray(X, F64) @ cast(W).T + exp[name + ".bias"][None, :]

    x = np.asarray(x, F64)
    hd = c.head_dim
    dq, dk = c.n_q * hd, c.n_kv * hd
    if not c.ffn_only:
        xn, _ = ob.rmsnorm(x, c.eps)
        X = xn * exp["attn_norm.gain"][None, :]
        Q = dlin("q", X, dq, c.d)
        K = dlin("k", X, dk, c.d)
        V = dlin("v", X, dk, c.d)
        cos, sin = ob.rope_tables(c.T, hd, c.rope_theta)
        O, _ = ob.attention(ob.rope(Q, c.n_q, hd, cos, sin), ob.rope(K, c.n_kv, hd, cos, sin), V,
                            c.n_q, c.n_kv, hd)
        h1 = x + dlin("o", O, c.d, dq)
        xn2, _ = ob.rmsnorm(h1, c.eps)
    else:
        h1, xn2 = None, x
    X2 = xn2 * exp["ffn_in.gain"][None, :]
    A = ob.silu(dlin("gate", X2, c.F, c.d)) * dlin("up", X2, c.F, c.d)
    D = dlin("down", A, c.d, c.F)
    return D if c.ffn_only else h1 + D
