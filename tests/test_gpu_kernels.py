"""GPU parity of the individual kernels against the CPU oracle, through the C ABI.

Integer results (codes, zero points, argmax/argmin) and the float32 code path
(step h, dequantized values) must match bit for bit: both sides evaluate the
same float32 operations in the same order with IEEE division and rint.
Reductions and products (bias fold, GEMM, backward sums) are compared by
relative Frobenius norm against the oracle's float64 results.
"""
import numpy as np
import pytest
import torch

import post_quantization_amd as omq
from oracle import quant
from oracle.ops import ExactOps
import synth
from gpu_util import DEV, bf16_np, dev, host, log, rel

pytestmark = pytest.mark.gpu

F32 = np.float32


def _params(rng, c_out, c_in):
    ag = rng.uniform(0.0, 6.0, c_out).astype(F32)
    ab = rng.uniform(0.0, 6.0, c_out).astype(F32)
    s = rng.uniform(0.5, 2.0, c_in).astype(F32)
    d = (rng.standard_normal(c_in) * 0.1).astype(F32)
    B = rng.standard_normal(c_out).astype(F32)
    return ag, ab, s, d, B


@pytest.mark.parametrize("c_out,c_in,nbits,let,out", [
    (77, 200, 4, True, "f32"), (64, 4096, 3, True, "bf16"), (16, 11008, 2, False, "bf16"),
    (130, 1028, 8, True, "f32"), (4096, 4096, 4, True, "bf16"), (24, 8200, 4, True, "f32"),
    (40, 28672, 2, True, "bf16")])
def test_lwc_fakequant_bitexact(c_out, c_in, nbits, let, out):
    log("lwc_fakequant", c_out, c_in, nbits, let, out)
    rng = np.random.default_rng(c_out + c_in)
    W = synth.normal(90, c_out, (c_out, c_in), synth.WEIGHT_STD)
    ag, ab, s, d, B = _params(rng, c_out, c_in)
    if not let:
        s = d = None
    ref = quant.lwc_fakequant(W, ag, ab, nbits, s, d, B)
    od = torch.float32 if out == "f32" else torch.bfloat16
    r = omq.lwc_fakequant(dev(W, torch.bfloat16), dev(ag), dev(ab), nbits,
                          dev(s) if let else None, dev(d) if let else None, dev(B),
                          out_dtype=od, want_bias=True, want_codes=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(r["arg_max"]), ref.st.iM)
    assert np.array_equal(host(r["arg_min"]), ref.st.im)
    assert np.array_equal(host(r["h"]), ref.h)
    assert np.array_equal(host(r["z"]), ref.z)
    assert np.array_equal(host(r["codes"]), ref.codes)
    expect = ref.W_hat if out == "f32" else bf16_np(ref.W_hat)
    assert np.array_equal(host(r["W_hat"]).astype(np.float64), np.asarray(expect, np.float64))
    assert rel(host(r["B_tilde"]), ref.B_tilde) < 1e-5


@pytest.mark.parametrize("c_out,c_in,nbits,let,wdt", [
    (40, 1024, 2, True, "bf16"), (96, 384, 3, False, "f32"), (4096, 4096, 4, True, "bf16"),
    (33, 11008, 3, True, "bf16")])
def test_lwc_group128_bitexact(c_out, c_in, nbits, let, wdt):
    """Group-wise LWC: per (row, 128-column group) logits, max/min, h, z and codes
    equal the oracle's bit for bit; arg_max / arg_min are columns of the row."""
    log("lwc_g128", c_out, c_in, nbits, let, wdt)
    rng = np.random.default_rng(c_out + 3 * c_in)
    G = c_in // 128
    W = synth.normal(94, c_out, (c_out, c_in), synth.WEIGHT_STD, bf16=(wdt == "bf16"))
    ag = rng.uniform(0.0, 6.0, c_out * G).astype(F32)
    ab = rng.uniform(0.0, 6.0, c_out * G).astype(F32)
    s = rng.uniform(0.5, 2.0, c_in).astype(F32) if let else None
    d = (rng.standard_normal(c_in) * 0.1).astype(F32) if let else None
    B = rng.standard_normal(c_out).astype(F32)
    ref = quant.lwc_fakequant(W, ag, ab, nbits, s, d, B, group=128)
    tdt = torch.bfloat16 if wdt == "bf16" else torch.float32
    r = omq.lwc_fakequant(dev(W, tdt), dev(ag), dev(ab), nbits, dev(s) if let else None,
                          dev(d) if let else None, dev(B), out_dtype=torch.float32,
                          want_bias=True, want_codes=True, group=128)
    torch.cuda.synchronize()
    base = (np.arange(c_out * G) % G) * 128
    assert np.array_equal(host(r["arg_max"]), ref.st.iM + base)
    assert np.array_equal(host(r["arg_min"]), ref.st.im + base)
    assert np.array_equal(host(r["h"]), ref.h)
    assert np.array_equal(host(r["z"]), ref.z)
    assert np.array_equal(host(r["codes"]), ref.codes)
    assert np.array_equal(host(r["W_hat"]), ref.W_hat)
    assert rel(host(r["B_tilde"]), ref.B_tilde) < 1e-5
    # straight-through backward, grouped (tile pass)
    g = (rng.standard_normal((c_out, c_in)) * 1e-3).astype(F32)
    v = rng.standard_normal(c_out).astype(F32)
    gWt, gg, gb = quant.lwc_bwd(g, ref)
    gam, bet = ref.st.gamma.astype(np.float64), ref.st.beta.astype(np.float64)
    ga, gbb, gs, gd = omq.lwc_backward(dev(g), dev(W, tdt), nbits, dev(ag), dev(ab), r["h"],
                                       r["z"], r["arg_max"], r["arg_min"],
                                       s=dev(s) if let else None, dy_colsum=dev(v),
                                       want_s=let, want_delta=True, group=128)
    torch.cuda.synchronize()
    assert rel(host(ga), gg * gam * (1 - gam)) < 1e-4
    assert rel(host(gbb), gb * bet * (1 - bet)) < 1e-4
    if let:
        assert rel(host(gs), np.sum(gWt * W.astype(np.float64), axis=0)) < 1e-4
    assert rel(host(gd), W.astype(np.float64).T @ v) < 1e-5


@pytest.mark.parametrize("T,C,nbits,mode,xdt", [
    (48, 200, 4, "div", "f32"), (33, 4096, 4, "div", "bf16"), (64, 4096, 8, "mul", "f32"),
    (40, 11008, 4, "none", "f32"), (2048, 4096, 4, "div", "bf16"), (24, 6000, 4, "div", "f32"),
    (16, 11008, 3, "mul", "bf16")])
def test_act_quant_bitexact(T, C, nbits, mode, xdt):
    log("act_quant", T, C, nbits, mode, xdt)
    rng = np.random.default_rng(T * 7 + C)
    X = synth.outlier_activations(91, T, T, C, max(1, C // 100), 20.0, 100.0, bf16=(xdt == "bf16"))
    if xdt == "f32":
        X = (X * rng.uniform(0.5, 1.5, X.shape)).astype(F32)
    s = rng.uniform(0.5, 2.0, C).astype(F32)
    d = (rng.standard_normal(C) * 0.3).astype(F32)
    ops = ExactOps(bf16=False)
    if mode == "div":
        Xt, lm = quant.let_act(X, s, d), omq.LET_DIV
    elif mode == "mul":
        Xt, lm, d = ops.mul(X, s), omq.LET_MUL, None
    else:
        Xt, lm, s, d = X, omq.LET_NONE, None, None
    st = quant.quantize_rows(Xt, F32(1), F32(1), nbits)
    r = omq.act_quant(dev(X, torch.float32 if xdt == "f32" else torch.bfloat16), nbits, lm,
                      dev(s) if s is not None else None, dev(d) if d is not None else None,
                      out_dtype=torch.float32, want_codes=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(r["codes"]), st.codes)
    assert np.array_equal(host(r["h"]), st.h)
    assert np.array_equal(host(r["z"]), st.z)
    assert np.array_equal(host(r["arg_max"]), st.iM)
    assert np.array_equal(host(r["X_hat"]), st.xhat)
    rb = omq.act_quant(dev(X, torch.float32 if xdt == "f32" else torch.bfloat16), nbits, lm,
                       dev(s) if s is not None else None, dev(d) if d is not None else None,
                       out_dtype=torch.bfloat16)
    assert np.array_equal(host(rb["X_hat"]).astype(np.float64), bf16_np(st.xhat))


def _near_tie_rows(rng, rows, cols, nbits):
    """Rows (in x~ space) whose quotients x~/h sit on, or within 3 ulp of, a
    half-integer: every element is a rounding decision that a quotient formed
    as x * (1/h), a few ulp off the true one, could get wrong."""
    Q = F32(2 ** nbits - 1)
    out = np.empty((rows, cols), F32)
    for r in range(rows):
        m, M = F32(-rng.uniform(0.5, 3.0)), F32(rng.uniform(0.5, 3.0))
        h = F32(F32(M - m) / Q)
        lo, hi = float(m / h), float(M / h)
        ks = np.arange(np.ceil(lo), np.floor(hi)) + 0.5
        ks = ks[(ks > lo + 0.5) & (ks < hi - 0.5)]
        y = (rng.choice(ks, cols).astype(F32) * h).astype(F32)
        steps = rng.integers(-3, 4, cols)
        for st in range(1, 4):
            y = np.where(steps >= st, np.nextafter(y, F32(np.inf)), y)
            y = np.where(steps <= -st, np.nextafter(y, F32(-np.inf)), y)
        y[0], y[1] = m, M
        out[r] = y[rng.permutation(cols)]
    return out


@pytest.mark.parametrize("nbits,mode,C", [(4, "none", 520), (2, "mul", 520), (4, "div", 520),
                                          (8, "div", 520), (4, "div", 4096), (4, "div", 6000),
                                          (3, "mul", 11008)])
def test_act_quant_near_ties(nbits, mode, C):
    log("act_quant_near_ties", nbits, mode, C)
    rng = np.random.default_rng(40 + nbits)
    T = 64
    Xt0 = _near_tie_rows(rng, T, C, nbits)
    s = rng.uniform(0.5, 2.0, C).astype(F32)
    d = (rng.standard_normal(C) * 0.3).astype(F32)
    ops = ExactOps(bf16=False)
    if mode == "none":
        X, lm, s, d = Xt0, omq.LET_NONE, None, None
        Xt = X
    elif mode == "mul":
        X, lm, d = (Xt0 / s).astype(F32), omq.LET_MUL, None
        Xt = ops.mul(X, s)
    else:
        X, lm = (Xt0 * s + d).astype(F32), omq.LET_DIV
        Xt = quant.let_act(X, s, d)
    st, _ = quant.act_quant(Xt, nbits)
    r = omq.act_quant(dev(X), nbits, lm, dev(s) if s is not None else None,
                      dev(d) if d is not None else None, out_dtype=torch.float32, want_codes=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(r["h"]), st.h)
    assert np.array_equal(host(r["codes"]), st.codes)
    assert np.array_equal(host(r["X_hat"]), st.xhat)
    # backward: dL/dx is gated element by element by the in-range decision
    g = rng.standard_normal((T, C)).astype(F32)
    gXt = quant.act_quant_bwd(g, st)
    gx, _, _ = omq.act_quant_backward(dev(g), dev(X), nbits, r["h"], r["z"], r["arg_max"],
                                      r["arg_min"], lm, dev(s) if s is not None else None,
                                      dev(d) if d is not None else None, want_gx=True)
    torch.cuda.synchronize()
    expect = gXt / s.astype(np.float64) if mode == "div" else (
        gXt * s.astype(np.float64) if mode == "mul" else gXt)
    err = np.abs(host(gx) - expect)
    assert np.all(err <= 1e-5 * (np.abs(expect) + 1.0))


@pytest.mark.parametrize("nbits,c_in", [(2, 1032), (3, 1032), (4, 1032), (4, 8200)])
def test_lwc_near_ties(nbits, c_in):
    """Weight side at gamma = beta = 1 (logits 30 give sigmoid exactly 1 in float32),
    LET scale s on the columns, float32 weights built so that s * W / h lands on
    or next to half-integers."""
    log("lwc_near_ties", nbits, c_in)
    rng = np.random.default_rng(50 + nbits)
    c_out = 48
    Wt0 = _near_tie_rows(rng, c_out, c_in, nbits)
    s = rng.uniform(0.5, 2.0, c_in).astype(F32)
    W = (Wt0 / s).astype(F32)
    ag = np.full(c_out, 30.0, F32)
    ab = np.full(c_out, 30.0, F32)
    ref = quant.lwc_fakequant(W, ag, ab, nbits, s, None, None)
    r = omq.lwc_fakequant(dev(W), dev(ag), dev(ab), nbits, dev(s), out_dtype=torch.float32,
                          want_codes=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(r["h"]), ref.h)
    assert np.array_equal(host(r["z"]), ref.z)
    assert np.array_equal(host(r["codes"]), ref.codes)
    assert np.array_equal(host(r["W_hat"]), ref.W_hat)


def test_act_quant_passthrough_and_let_apply():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((24, 64)).astype(F32)
    W = synth.normal(92, 1, (40, 64), 0.02)
    s = rng.uniform(0.5, 2.0, 64).astype(F32)
    d = rng.standard_normal(64).astype(F32)
    B = rng.standard_normal(40).astype(F32)
    r = omq.act_quant(dev(X), 16, omq.LET_DIV, dev(s), dev(d), out_dtype=torch.float32)
    assert np.array_equal(host(r["X_hat"]), quant.let_act(X, s, d))
    Xt, Wt, Bt = omq.let_apply(dev(s), dev(d), X=dev(X), W=dev(W, torch.bfloat16), B=dev(B),
                               want_bias=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(Xt), quant.let_act(X, s, d))
    assert np.array_equal(host(Wt), quant.let_weight(W, s))
    assert rel(host(Bt), quant.bias_fold(W, B, d)) < 1e-5


@pytest.mark.parametrize("M,N,K,dt,ta,tb", [
    (200, 136, 328, "bf16", 0, 0), (128, 256, 64, "bf16", 0, 0), (2048, 4096, 4096, "bf16", 0, 0),
    (70, 50, 36, "f32", 0, 0), (2048, 12288, 4096, "bf16", 0, 0),
    (4096, 8192, 512, "bf16", 0, 0), (256, 256, 4104, "bf16", 0, 0),
    (200, 136, 328, "bf16", 0, 1), (200, 136, 328, "bf16", 1, 0), (200, 136, 328, "bf16", 1, 1),
    (2048, 4096, 2048, "bf16", 1, 1), (2048, 4096, 11008, "bf16", 0, 1),
    (4096, 8192, 512, "bf16", 1, 0), (4096, 8192, 256, "bf16", 0, 1),
    (4096, 8192, 320, "bf16", 1, 1), (384, 640, 192, "bf16", 1, 1),
    (70, 50, 36, "f32", 1, 1)])
def test_gemm(M, N, K, dt, ta, tb):
    log("gemm", M, N, K, dt, ta, tb)
    rng = np.random.default_rng(M + N + K)
    A = rng.standard_normal((M, K)).astype(F32)
    B = rng.standard_normal((N, K)).astype(F32)
    bias = rng.standard_normal(N).astype(F32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        A, B = synth.to_bf16(A), synth.to_bf16(B)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    C = omq.gemm(dev(As, tdt), dev(Bs, tdt), bias=dev(bias), trans_a=bool(ta), trans_b=bool(tb))
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 256 else rng.choice(M, 96, replace=False)
    ref = A[rows].astype(np.float64) @ B.astype(np.float64).T + bias
    assert rel(host(C)[rows], ref) < 2e-5
    # accumulate into the previous result
    C2 = omq.gemm(dev(As, tdt), dev(Bs, tdt), C=C, accumulate=True, alpha=0.5, trans_a=bool(ta),
                  trans_b=bool(tb))
    torch.cuda.synchronize()
    assert rel(host(C2)[rows], 1.5 * (A[rows].astype(np.float64) @ B.astype(np.float64).T) + bias) < 2e-5


@pytest.mark.parametrize("M,N,K,abits,wbits", [
    (256, 384, 4096, 4, 4),       # whole tiles: direct LDS copies
    (200, 136, 1376, 4, 3),       # ragged rows, columns and k-steps: register staging
    (512, 768, 11008, 7, 4),      # the FFN down width, 7-bit codes
    (2048, 1024, 512, 4, 2)])
def test_code_gemm(M, N, K, abits, wbits):
    """The product on integer codes against the oracle's code product, with the codes,
    steps and zero points the oracle's quantizers give for synthetic activations
    (a few all-positive token rows, whose zero point lies below the code range) and
    LWC weights; the code sums through omq_code_rowsum, bit for bit against numpy.
    The kernel's integer sum is exact and rounded once, so the bound is a float32
    rounding of the result and of the bias addition."""
    log("code_gemm", M, N, K, abits, wbits)
    rng = np.random.default_rng(M + N + K)
    X = synth.normal(91, M, (M, K), 1.0)
    X[::37] += 6.0
    W = synth.normal(92, N, (N, K), synth.WEIGHT_STD)
    sx, _ = quant.act_quant(X, abits)
    ag, ab, _, _, B = _params(rng, N, K)
    wq = quant.lwc_fakequant(W, ag, ab, wbits)
    assert (sx.z < 0).any()
    qa, qb = dev(sx.codes, torch.uint8), dev(wq.codes, torch.uint8)
    sa, sb = omq.code_rowsum(qa), omq.code_rowsum(qb)
    assert np.array_equal(host(sa), sx.codes.astype(np.int64).sum(1))
    assert np.array_equal(host(sb), wq.codes.astype(np.int64).sum(1))
    C = omq.code_gemm(qa, dev(sx.h), dev(sx.z), qb, dev(wq.h), dev(wq.z), sa, sb, bias=dev(B))
    torch.cuda.synchronize()
    want = quant.code_product(sx.codes, sx.h, sx.z, wq.codes, wq.h, wq.z, B)
    got = host(C).astype(np.float64)
    err = np.abs(got - want)
    # (plus the oracle's own float64 summation error, relative to sum |terms|)
    absa = np.abs(sx.codes - sx.z[:, None]) * sx.h[:, None]
    absb = np.abs(wq.codes - wq.z[:, None]) * wq.h[:, None]
    bound = 2.0 ** -23 * (np.abs(want - B[None, :]) + 2 * np.abs(B)[None, :]) + \
        2.0 ** -40 * (absa @ absb.T) + 1e-30
    log("max err / bound %.3f" % (err / bound).max())
    assert (err <= bound).all()


def _pack4(codes):
    """Two 4-bit codes to a byte, code k of a row in byte k // 2, the low nibble for even
    k (numpy, from the definition)."""
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("M,N,K,abits,wbits", [
    (256, 384, 4096, 4, 4),       # the 7B widths
    (128, 256, 11008, 4, 3),      # the FFN down width
    (2048, 1024, 512, 4, 2)])
def test_code_gemm4_packed(M, N, K, abits, wbits):
    """The product on 4-bit codes stored two to a byte equals the product on byte codes
    bit for bit (the same integer sums, unpacked inside the kernel, and the same single
    rounding), and the oracle's code product within a float32 rounding."""
    log("code_gemm4", M, N, K, abits, wbits)
    rng = np.random.default_rng(M + N + K + 4)
    X = synth.normal(94, M, (M, K), 1.0)
    X[::37] += 6.0
    W = synth.normal(95, N, (N, K), synth.WEIGHT_STD)
    sx, _ = quant.act_quant(X, abits)
    ag, ab, _, _, B = _params(rng, N, K)
    wq = quant.lwc_fakequant(W, ag, ab, wbits)
    assert sx.codes.max() < 16 and wq.codes.max() < 16
    qa, qb = dev(sx.codes, torch.uint8), dev(wq.codes, torch.uint8)
    sa, sb = omq.code_rowsum(qa), omq.code_rowsum(qb)
    pa, pb = dev(_pack4(sx.codes), torch.uint8), dev(_pack4(wq.codes), torch.uint8)
    C1 = omq.code_gemm(qa, dev(sx.h), dev(sx.z), qb, dev(wq.h), dev(wq.z), sa, sb, bias=dev(B))
    C4 = omq.code_gemm4(pa, dev(sx.h), dev(sx.z), pb, dev(wq.h), dev(wq.z), K, sa, sb,
                        bias=dev(B))
    torch.cuda.synchronize()
    got1, got4 = host(C1), host(C4)
    assert np.array_equal(got4.view(np.uint32), got1.view(np.uint32))
    want = quant.code_product(sx.codes, sx.h, sx.z, wq.codes, wq.h, wq.z, B)
    assert rel(got4.astype(np.float64), want) < 1e-6


@pytest.mark.parametrize("c_out,c_in,nbits,let", [(77, 200, 4, True), (96, 4096, 2, True),
                                                  (64, 11008, 3, False), (4096, 4096, 4, True)])
def test_lwc_backward(c_out, c_in, nbits, let):
    log("lwc_backward", c_out, c_in, nbits, let)
    rng = np.random.default_rng(c_out * 3 + c_in)
    W = synth.normal(93, c_out, (c_out, c_in), synth.WEIGHT_STD)
    ag, ab, s, d, B = _params(rng, c_out, c_in)
    if not let:
        s = None
    ref = quant.lwc_fakequant(W, ag, ab, nbits, s, None, None)
    g = (rng.standard_normal((c_out, c_in)) * 1e-3).astype(F32)
    v = rng.standard_normal(c_out).astype(F32)
    gWt, gg, gb = quant.quantize_rows_bwd(g, ref.st)
    gam, bet = ref.st.gamma.astype(np.float64), ref.st.beta.astype(np.float64)
    r = omq.lwc_fakequant(dev(W, torch.bfloat16), dev(ag), dev(ab), nbits,
                          dev(s) if let else None, out_dtype=torch.bfloat16)
    ga, gbb, gs, gd = omq.lwc_backward(dev(g), dev(W, torch.bfloat16), nbits, dev(ag), dev(ab),
                                       r["h"], r["z"], r["arg_max"], r["arg_min"],
                                       s=dev(s) if let else None, dy_colsum=dev(v),
                                       want_s=let, want_delta=True)
    torch.cuda.synchronize()
    assert rel(host(ga), gg * gam * (1 - gam)) < 1e-4
    assert rel(host(gbb), gb * bet * (1 - bet)) < 1e-4
    if let:
        assert rel(host(gs), np.sum(gWt * W.astype(np.float64), axis=0)) < 1e-4
    assert rel(host(gd), W.astype(np.float64).T @ v) < 1e-5


@pytest.mark.parametrize("T,C,nbits,mode", [(48, 200, 4, "div"), (64, 4096, 4, "div"),
                                            (64, 4096, 8, "mul"), (40, 11008, 4, "none"),
                                            (2048, 4096, 4, "div"), (32, 512, 16, "div")])
def test_act_quant_backward(T, C, nbits, mode):
    log("act_quant_backward", T, C, nbits, mode)
    rng = np.random.default_rng(T + 5 * C)
    X = (rng.standard_normal((T, C)) * rng.uniform(0.2, 3.0, C)).astype(F32)
    s = rng.uniform(0.5, 2.0, C).astype(F32)
    d = (rng.standard_normal(C) * 0.3).astype(F32)
    ops = ExactOps(bf16=False)
    lm = {"div": omq.LET_DIV, "mul": omq.LET_MUL, "none": omq.LET_NONE}[mode]
    if mode == "div":
        Xt = quant.let_act(X, s, d)
    elif mode == "mul":
        Xt, d = ops.mul(X, s), None
    else:
        Xt, s, d = X, None, None
    st, _ = quant.act_quant(Xt, nbits)
    g = rng.standard_normal((T, C)).astype(F32)
    gXt = quant.act_quant_bwd(g, st)
    Xt64 = Xt.astype(np.float64)
    r = omq.act_quant(dev(X), nbits, lm, dev(s) if s is not None else None,
                      dev(d) if d is not None else None, out_dtype=torch.float32)
    gx, gs, gd = omq.act_quant_backward(
        dev(g), dev(X), nbits, r["h"], r["z"], r["arg_max"], r["arg_min"], lm,
        dev(s) if s is not None else None, dev(d) if d is not None else None,
        want_gx=True, want_s=mode != "none", want_delta=mode == "div")
    torch.cuda.synchronize()
    if mode == "div":
        s64 = s.astype(np.float64)
        assert rel(host(gx), gXt / s64) < 1e-5
        assert rel(host(gs), np.sum(gXt * (-Xt64 / s64), axis=0)) < 1e-4
        assert rel(host(gd), np.sum(gXt, axis=0) * (-1 / s64)) < 1e-4
    elif mode == "mul":
        assert rel(host(gx), gXt * s.astype(np.float64)) < 1e-5
        assert rel(host(gs), np.sum(gXt * X.astype(np.float64), axis=0)) < 1e-4
    else:
        assert rel(host(gx), gXt) < 1e-5


def test_optimizers():
    """AdamW / SGD against the oracle's float64 update rounded to float32: the new
    parameters agree to 2 float32 ulps, the moments to 1e-6 relative."""
    from oracle import optim
    rng = np.random.default_rng(9)
    n, n_lwc = 1000, 600
    th = rng.standard_normal(n).astype(F32)
    g = (rng.standard_normal(n) * 1e-2).astype(F32)
    m = (rng.standard_normal(n) * 1e-3).astype(F32)
    v = (rng.uniform(0, 1e-4, n)).astype(F32)
    tt, tg, tm, tv = dev(th), dev(g), dev(m), dev(v)
    omq.adamw(tt, tg, tm, tv, n_lwc, 5e-3, 1e-2, 3)
    torch.cuda.synchronize()
    e1 = optim.adamw(th[:n_lwc], g[:n_lwc], m[:n_lwc], v[:n_lwc], 3, 5e-3)
    e2 = optim.adamw(th[n_lwc:], g[n_lwc:], m[n_lwc:], v[n_lwc:], 3, 1e-2)
    expect = np.concatenate([e1[0], e2[0]])
    lr = np.where(np.arange(n) < n_lwc, 5e-3, 1e-2)
    # 2 ulp of the parameter plus the float32 rounding of the update itself (~lr)
    assert np.all(np.abs(host(tt) - expect) <= 2 * np.spacing(np.abs(expect)) + 1e-5 * lr)
    assert rel(host(tm), np.concatenate([e1[1], e2[1]])) < 1e-6
    assert rel(host(tv), np.concatenate([e1[2], e2[2]])) < 1e-6
    tt = dev(th)
    omq.sgd(tt, tg, n_lwc, 5e-3, 1e-2)
    torch.cuda.synchronize()
    expect = np.concatenate([optim.sgd(th[:n_lwc], g[:n_lwc], 5e-3),
                             optim.sgd(th[n_lwc:], g[n_lwc:], 1e-2)])
    assert np.all(np.abs(host(tt) - expect) <= 2 * np.spacing(np.abs(expect)) + 1e-5 * lr * 1e-2)


@pytest.mark.parametrize("C,xdt", [(520, "f32"), (4096, "f32"), (6000, "f32"), (4096, "bf16")])
def test_act_quant_degenerate_rows(C, xdt):
    """Rows the quantizer treats specially: constant rows (max = min, the step floored
    at 1e-8), all-zero rows, a single spike, ties for the max and min (first index
    wins), a row whose range is one float32 ulp; bit-exact against the oracle on every
    kernel that row width takes."""
    log("act_quant_degenerate", C, xdt)
    rng = np.random.default_rng(C)
    T = 12
    X = np.zeros((T, C), F32)
    X[0] = 3.25
    X[1] = -0.5
    X[3, C // 3] = 7.0
    X[4] = rng.standard_normal(C).astype(F32)
    X[4, [5, C - 7]] = 9.0
    X[4, [2, C - 3]] = -9.0
    X[5] = np.float32(1.0)
    X[5, C // 2] = np.nextafter(F32(1.0), F32(2.0))
    X[6] = rng.standard_normal(C).astype(F32) * F32(1e-30)
    X[7:] = rng.standard_normal((T - 7, C)).astype(F32)
    if xdt == "bf16":
        X = bf16_np(X).astype(F32)
    for nbits in (2, 4, 8):
        st = quant.quantize_rows(X, F32(1), F32(1), nbits)
        r = omq.act_quant(dev(X, torch.float32 if xdt == "f32" else torch.bfloat16), nbits,
                          omq.LET_NONE, None, None, out_dtype=torch.float32, want_codes=True)
        torch.cuda.synchronize()
        assert np.array_equal(host(r["h"]), st.h), nbits
        assert np.array_equal(host(r["z"]), st.z), nbits
        assert np.array_equal(host(r["arg_max"]), st.iM), nbits
        assert np.array_equal(host(r["arg_min"]), st.im), nbits
        assert np.array_equal(host(r["codes"]), st.codes), nbits
        assert np.array_equal(host(r["X_hat"]), st.xhat), nbits


@pytest.mark.parametrize("c_in", [520, 4096, 11008])
def test_lwc_degenerate_rows(c_in):
    """Weight rows the quantizer treats specially (constant, all-zero, a single spike,
    tied extremes, a one-ulp range), with gamma = beta (a constant row then has a zero
    range, the step floored at 1e-8) and with gamma != beta; bit-exact against the
    oracle on every row kernel that width takes."""
    log("lwc_degenerate", c_in)
    rng = np.random.default_rng(c_in + 1)
    c_out = 8
    W = np.zeros((c_out, c_in), F32)
    W[0] = 0.25
    W[1] = -0.125
    W[3, c_in // 3] = 0.5
    W[4] = (rng.standard_normal(c_in) * 0.02).astype(F32)
    W[4, [5, c_in - 7]] = 0.3
    W[4, [2, c_in - 3]] = -0.3
    W[5] = 1.0
    W[5, c_in // 2] = np.nextafter(F32(1.0), F32(2.0))
    W[6:] = (rng.standard_normal((c_out - 6, c_in)) * 0.02).astype(F32)
    W = bf16_np(W).astype(F32)
    for same in (True, False):
        ag = np.full(c_out, 4.0, F32)
        ab = ag.copy() if same else rng.uniform(0.0, 6.0, c_out).astype(F32)
        for nbits in (2, 4):
            ref = quant.lwc_fakequant(W, ag, ab, nbits, None, None, None)
            r = omq.lwc_fakequant(dev(W, torch.bfloat16), dev(ag), dev(ab), nbits,
                                  out_dtype=torch.float32, want_codes=True)
            torch.cuda.synchronize()
            assert np.array_equal(host(r["h"]), ref.h), (same, nbits)
            assert np.array_equal(host(r["z"]), ref.z), (same, nbits)
            assert np.array_equal(host(r["codes"]), ref.codes), (same, nbits)
            assert np.array_equal(host(r["W_hat"]), ref.W_hat), (same, nbits)


@pytest.mark.parametrize("kind,rows,cols,dt", [
    ("act", 64, 200, "f32"), ("act", 64, 1024, "bf16"), ("act", 40, 4096, "f32"),
    ("act", 24, 11008, "bf16"), ("act", 16, 6000, "f32"),
    ("lwc", 48, 4096, "bf16"), ("lwc", 33, 1032, "bf16"), ("lwc_g128", 40, 1024, "bf16")])
def test_nonfinite_flag(kind, rows, cols, dt):
    """The input-health flag: a row holding one NaN and a row holding one infinity set
    it (every quantizer kernel variant: the widths pick them); every other row's
    codes, dequantized values, h, z and extreme-value columns are bit-identical to
    those of the same input with the two rows made finite, which leaves the flag at
    zero; the bad rows' extreme-value columns still name columns of their row."""
    log("nonfinite", kind, rows, cols, dt)
    rng = np.random.default_rng(rows + cols)
    X = (rng.standard_normal((rows, cols)) * 0.5).astype(F32)
    if dt == "bf16":
        X = synth.to_bf16(X)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    bad = X.copy()
    bad[3, cols // 3] = np.nan
    bad[7, cols - 1] = np.inf
    group = 128 if kind == "lwc_g128" else 0
    nrows = rows * (cols // 128 if group else 1)
    ag = dev(rng.uniform(2.0, 5.0, nrows).astype(F32))
    ab = dev(rng.uniform(2.0, 5.0, nrows).astype(F32))
    s = dev(rng.uniform(0.7, 1.4, cols).astype(F32))

    def run(A):
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        if kind == "act":
            r = omq.act_quant(dev(A, tdt), 4, omq.LET_DIV, s, None, want_codes=True,
                              nonfinite=flag)
            out = (r["X_hat"], r["h"], r["z"], r["arg_max"], r["arg_min"], r["codes"])
        else:
            r = omq.lwc_fakequant(dev(A, tdt), ag, ab, 3, s, out_dtype=torch.bfloat16,
                                  want_codes=True, group=group, nonfinite=flag)
            out = (r["W_hat"], r["h"], r["z"], r["arg_max"], r["arg_min"], r["codes"])
        torch.cuda.synchronize()
        return int(host(flag)[0]), [host(t) for t in out]

    f_good, good = run(X)
    f_bad, badr = run(bad)
    assert f_good == 0 and f_bad == 1
    ok = np.ones(rows, bool)
    ok[[3, 7]] = False
    per = cols // 128 if group else 1
    okq = np.repeat(ok, per)
    for name, a, b in zip(("x_hat", "h", "z", "arg_max", "arg_min", "codes"), good, badr):
        sel = okq if a.ndim == 1 else ok
        assert np.array_equal(np.asarray(a)[sel], np.asarray(b)[sel]), name
    for am in (badr[3], badr[4]):
        assert ((am >= 0) & (am < cols)).all()
