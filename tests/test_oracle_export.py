"""Pins of the deployment-form oracle (oracle/export.py): the packed layout, the
LET folds and the weight-only product from packed codes."""
import numpy as np
import pytest

from oracle import export as ex
from oracle import quant

F32 = np.float32
F64 = np.float64


@pytest.mark.parametrize("nbits", [2, 3, 4, 8])
def test_pack_roundtrip(nbits):
    rng = np.random.default_rng(nbits)
    for C in (1, 7, 32, 130, 1000):
        codes = rng.integers(0, 2 ** nbits, (5, C)).astype(np.uint8)
        words = ex.pack_codes(codes, nbits)
        assert words.dtype == np.uint32
        assert words.shape == (5, -(-C // (32 // nbits)))
        assert np.array_equal(ex.unpack_codes(words, nbits, C), codes)


def test_pack_hand_built_words():
    # 4 bit: codes 1..8 -> 0x87654321 (lowest column in the lowest nibble)
    w = ex.pack_codes(np.array([[1, 2, 3, 4, 5, 6, 7, 8]], np.uint8), 4)
    assert w.tolist() == [[0x87654321]]
    # 3 bit: 10 codes per word, two high bits unused; codes all 7 -> 2^30 - 1
    w = ex.pack_codes(np.full((1, 10), 7, np.uint8), 3)
    assert w.tolist() == [[(1 << 30) - 1]]
    # 2 bit: a partial word is zero-padded
    w = ex.pack_codes(np.array([[3, 0, 1]], np.uint8), 2)
    assert w.tolist() == [[0b01_00_11]]


def test_dequant_matches_fakequant():
    """(q - z) h from the codes is the fake-quant output, per channel and per group."""
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((12, 256)) * 0.02).astype(F32)
    for group, rows in ((None, 12), (128, 24)):
        ag = rng.uniform(1, 5, rows).astype(F32)
        ab = rng.uniform(1, 5, rows).astype(F32)
        r = quant.lwc_fakequant(W, ag, ab, 4, group=group)
        assert np.array_equal(ex.dequant(r.codes, r.h, r.z, group), r.W_hat)


def test_fold_input_site_is_the_let_layer():
    """Weight-only: (X / s) W_hat^T + bias' equals X~ W_hat^T + B~ (float64)."""
    rng = np.random.default_rng(4)
    X = rng.standard_normal((6, 40))
    W_hat = rng.standard_normal((9, 40))
    B_t = rng.standard_normal(9)
    s = rng.uniform(0.5, 2.0, 40)
    d = rng.standard_normal(40)
    gain, bias = ex.fold_input_site(W_hat, B_t, s, d)
    ref = ((X - d) / s) @ W_hat.T + B_t
    assert np.allclose((X * gain) @ W_hat.T + bias, ref, rtol=1e-12, atol=1e-12)


def test_fold_value_site_through_attention():
    """P ((V - delta_o) / s_o) = P (V h / s_o scale) + (b - delta_o) / s_o when rows
    of P sum to one: fold the pair into the value projection's scales and bias."""
    rng = np.random.default_rng(5)
    T, C, dv = 7, 16, 8
    X = rng.standard_normal((T, C))
    codes = rng.integers(0, 16, (dv, C)).astype(F64)
    h = rng.uniform(0.01, 0.1, dv)
    z = rng.integers(0, 16, dv).astype(F64)
    b = rng.standard_normal(dv)
    s_o = rng.uniform(0.5, 2.0, dv)
    d_o = rng.standard_normal(dv)
    P = rng.uniform(0, 1, (T, T))
    P /= P.sum(axis=1, keepdims=True)
    V = X @ ((codes - z[:, None]) * h[:, None]).T + b
    ref = P @ ((V - d_o) / s_o)
    h2, b2 = ex.fold_value_site(h, b, s_o, d_o)
    V2 = X @ ((codes - z[:, None]) * h2[:, None]).T + b2
    assert np.allclose(P @ V2, ref, rtol=1e-12, atol=1e-12)


def test_wa16_linear_matches_fakequant_product():
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((20, 256)) * 0.02).astype(F32)
    X = quant.bf16(rng.standard_normal((3, 256)))
    ag = rng.uniform(1, 5, 40).astype(F32)
    ab = rng.uniform(1, 5, 40).astype(F32)
    r = quant.lwc_fakequant(W, ag, ab, 4, group=128)
    words = ex.pack_codes(r.codes, 4)
    Y = ex.wa16_linear(X, words, r.h, r.z, 4, 256, group=128)
    assert np.allclose(Y, X @ quant.bf16(r.W_hat).T, rtol=0, atol=0)


@pytest.mark.parametrize("kind", ["mha", "gqa_g8", "ffn"])
def test_exported_block_reproduces_the_calibrated_forward(kind):
    """Weight-only: the block rebuilt from packed codes, folded biases and gains,
    with no LET operators left, gives the calibration forward's output (exact
    float64 products on both sides; the only difference is X~'s float32 rounding
    in the calibration path)."""
    import synth
    from oracle import block as ob
    from oracle.ops import ExactOps
    c = {"mha": synth.BlockCfg(cfg=4, T=9, d=16, n_q=2, n_kv=2, F=24, wbits=4, abits=16,
                               head_dim=8, n_out=2, out_lo=5.0, out_hi=10.0),
         "gqa_g8": synth.BlockCfg(cfg=4, T=9, d=16, n_q=4, n_kv=2, F=24, wbits=3, abits=16,
                                  head_dim=8, n_out=2, out_lo=5.0, out_hi=10.0, group=8),
         "ffn": synth.BlockCfg(cfg=3, T=9, d=16, n_q=2, n_kv=2, F=24, wbits=2, abits=16,
                               head_dim=8, ffn_only=True, n_out=2, out_lo=5.0,
                               out_hi=10.0)}[kind]
    rng = np.random.default_rng(8)
    inp = synth.block_inputs(c)
    Wd = {k: v for k, v in inp.items() if k.startswith("W_")}
    shapes = synth.block_weight_shapes(c)
    th = ob.init_theta(c, shapes)
    for k in th:
        if k.startswith("a_"):
            th[k] = rng.uniform(0.5, 4.0, th[k].size).astype(F32)
        elif k.startswith("s"):
            th[k] = rng.uniform(0.6, 1.6, th[k].size).astype(F32)
        else:
            th[k] = (rng.standard_normal(th[k].size) * 0.2).astype(F32)
    y_cal, _ = ob.forward(c, inp["x"], Wd, th, ExactOps(bf16=False))
    exp = ex.export_block(c, Wd, th)
    y_dep = ex.deployed_forward(c, inp["x"], exp)
    assert np.max(np.abs(y_dep - y_cal)) <= 1e-5 * np.max(np.abs(y_cal))
    # and the fold is not vacuous: without the gain the block's update changes
    upd = y_cal - (0 if c.ffn_only else np.asarray(inp["x"], np.float64))
    bad = dict(exp)
    bad["ffn_in.gain"] = np.ones_like(exp["ffn_in.gain"])
    assert np.max(np.abs(ex.deployed_forward(c, inp["x"], bad) - y_cal)) > 1e-2 * np.max(
        np.abs(upd))
