"""GPU parity of the deployment form against the oracle (oracle/export.py),
through the C ABI: packing of the calibrated codes (bit-exact), the weight-only
LET folds, and the product on packed 4-bit codes, per output channel and with
128-channel groups, for token counts from single-token decode to a few tiles."""
import numpy as np
import pytest
import torch

import post_quantization_amd as omq
from oracle import export as ex
from oracle import quant
import synth
from gpu_util import DEV, dev, host, log, rel

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.mark.parametrize("nbits,cols", [(4, 4096), (4, 100), (2, 1000), (3, 517), (8, 36)])
def test_pack_codes_bitexact(nbits, cols):
    log("pack", nbits, cols)
    rng = np.random.default_rng(nbits * 1000 + cols)
    codes = rng.integers(0, 2 ** nbits, (37, cols)).astype(np.uint8)
    words = omq.pack_codes(torch.from_numpy(codes).cuda(), nbits)
    torch.cuda.synchronize()
    got = host(words).view(np.uint32)
    assert np.array_equal(got, ex.pack_codes(codes, nbits))


def _calibrated_layer(N, K, group, nbits, rng, let=True):
    """Synthetic weights through the GPU fake quantizer (codes, h, z) and the oracle's."""
    W = synth.normal(95, N + K, (N, K), synth.WEIGHT_STD)
    rows = N * (K // group if group else 1)
    ag = rng.uniform(1.0, 5.0, rows).astype(F32)
    ab = rng.uniform(1.0, 5.0, rows).astype(F32)
    s = rng.uniform(0.5, 2.0, K).astype(F32) if let else None
    ref = quant.lwc_fakequant(W, ag, ab, nbits, s, group=group or None)
    r = omq.lwc_fakequant(dev(W, torch.bfloat16), dev(ag), dev(ab), nbits,
                          dev(s) if let else None, out_dtype=torch.bfloat16, want_codes=True,
                          group=group)
    torch.cuda.synchronize()
    assert np.array_equal(host(r["codes"]), ref.codes)
    return W, s, ref, r


@pytest.mark.parametrize("N,K,group", [(96, 4096, 128), (300, 1024, 0), (4096, 4096, 128)])
def test_fold_linear(N, K, group):
    log("fold", N, K, group)
    rng = np.random.default_rng(N + K)
    W, s, ref, r = _calibrated_layer(N, K, group, 4, rng)
    words = omq.pack_codes(r["codes"], 4)
    delta = (rng.standard_normal(K) * 0.1).astype(F32)
    Bt = rng.standard_normal(N).astype(F32)
    s_o = rng.uniform(0.5, 2.0, N).astype(F32)
    d_o = (rng.standard_normal(N) * 0.1).astype(F32)
    W_hat = ex.dequant(ref.codes, ref.h, ref.z, group or None)
    # input site only
    b1, _ = omq.fold_linear(words, 4, N, K, r["h"], r["z"], group, dev(Bt), dev(s), dev(delta))
    _, eb1 = ex.fold_input_site(W_hat, Bt, s, delta)
    # input site, then the attention-output pair folded into this (value) projection
    b2, h2 = omq.fold_linear(words, 4, N, K, r["h"], r["z"], group, dev(Bt), dev(s), dev(delta),
                             dev(s_o), dev(d_o))
    torch.cuda.synchronize()
    G = K // group if group else 1
    eh2, eb2 = ex.fold_value_site(ref.h.reshape(N, G), eb1[:, None], s_o[:, None],
                                  d_o[:, None])
    assert rel(host(b1), eb1) < 1e-5
    assert rel(host(b2), eb2[:, 0]) < 1e-5
    assert np.allclose(host(h2).reshape(N, G), eh2, rtol=2 ** -23, atol=0)


@pytest.mark.parametrize("T,N,K,group", [(1, 4096, 4096, 128), (7, 300, 4096, 128),
                                         (32, 1024, 11008, 128), (100, 512, 1024, 0),
                                         (16, 22016, 4096, 128),
                                         # the vector-unit kernel at 1 to 3 tokens with
                                         # ragged N, per-channel steps and a tail
                                         # column position (K 11008)
                                         (1, 1000, 11008, 128), (2, 300, 1024, 0),
                                         (3, 1030, 4096, 128)])
def test_w4a16_gemm(T, N, K, group):
    log("w4a16", T, N, K, group)
    rng = np.random.default_rng(T * 7 + N + K)
    W, s, ref, r = _calibrated_layer(N, K, group, 4, rng, let=False)
    words = omq.pack_codes(r["codes"], 4)
    X = synth.to_bf16(rng.standard_normal((T, K)).astype(F32))
    bias = rng.standard_normal(N).astype(F32)
    Y = omq.w4a16_gemm(dev(X, torch.bfloat16), words, N, r["h"], r["z"], group, dev(bias))
    torch.cuda.synchronize()
    expect = ex.wa16_linear(X, ex.pack_codes(ref.codes, 4), ref.h, ref.z, 4, K,
                            group or None, bias)
    assert rel(host(Y), expect) < 1e-5
    # the same product through the fake-quant weight and the matrix-core GEMM
    Y2 = omq.gemm(dev(X, torch.bfloat16), r["W_hat"], bias=dev(bias))
    torch.cuda.synchronize()
    assert rel(host(Y), host(Y2)) < 1e-5


@pytest.mark.parametrize("kind", ["gqa_w4a16g128", "mha_w3a16", "ffn_w2a16g128"])
def test_export_block(kind):
    """The exported weight-only block (packed codes, (h, z), folded biases, gains)
    against the oracle's export of the same calibrated parameters."""
    from oracle import block as ob
    from post_quantization_amd import export
    c = {"gqa_w4a16g128": synth.reduced(synth.BLOCK_CFG4_W3G128, wbits=4, d=512, n_q=4,
                                        n_kv=2, F=1408),
         "mha_w3a16": synth.reduced(synth.BLOCK_CFG4_W3G128, group=0, d=384, n_q=3, n_kv=3,
                                    F=1032),
         "ffn_w2a16g128": synth.reduced(synth.FFN_CFG3_W2, group=128, d=512, F=1408)}[kind]
    log("export", kind)
    rng = np.random.default_rng(12)
    shapes = synth.block_weight_shapes(c)
    inp = synth.block_inputs(c)
    Wd = {k: v for k, v in inp.items() if k.startswith("W_")}
    th = ob.init_theta(c, shapes)
    for k in th:
        if k.startswith("a_"):
            th[k] = rng.uniform(1.0, 5.0, th[k].size).astype(F32)
        elif k.startswith("s"):
            th[k] = rng.uniform(0.7, 1.4, th[k].size).astype(F32)
        else:
            th[k] = (rng.standard_normal(th[k].size) * 0.05).astype(F32)
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group)
    W = [dev(Wd["W_" + n], torch.bfloat16) if ("W_" + n) in Wd else None
         for n in synth.WEIGHT_NAMES]
    got = export.export_block(d, W, dev(ob.pack(c, shapes, th)))
    torch.cuda.synchronize()
    want = ex.export_block(c, Wd, th)
    assert set(got) == set(want)
    for k, v in want.items():
        g = host(got[k])
        if k.endswith(".words"):
            assert np.array_equal(g.view(np.uint32), v), k
        elif k.endswith(".z") or (k.endswith(".h") and not k.startswith("v.")):
            assert np.array_equal(g, v.astype(F32)), k
        elif k.endswith(".bias"):
            assert rel(g, v) < 1e-5, k
        else:                        # v.h (divided by s_o) and the gains 1/s
            assert np.allclose(g, v, rtol=2 ** -23, atol=0), k


def test_w4a16_gemm_graph_replays():
    """The packed-code product captured into a HIP graph (as a decode loop replays
    it): every replay, with eager work and synchronizations in between, equals the
    eager result bit for bit, for the vector-unit (T = 1) and matrix-core (T = 16)
    kernels."""
    rng = np.random.default_rng(5)
    cases = []
    for T, N, K in ((1, 1024, 4096), (16, 512, 2048)):
        W, s, ref, r = _calibrated_layer(N, K, 128, 4, rng, let=False)
        words = omq.pack_codes(r["codes"], 4)
        X = dev(synth.to_bf16(rng.standard_normal((T, K)).astype(F32)), torch.bfloat16)
        Y = torch.empty(T, N, dtype=torch.float32, device=DEV)
        eager = omq.w4a16_gemm(X, words, N, r["h"], r["z"], 128).clone()
        cases.append((X, words, N, r["h"], r["z"], Y, eager))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for X, words, N, h, z, Y, _ in cases:
            omq.w4a16_gemm(X, words, N, h, z, 128, None, Y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for X, words, N, h, z, Y, _ in cases:
            omq.w4a16_gemm(X, words, N, h, z, 128, None, Y)
    for rep in range(3):
        for _, _, _, _, _, Y, _ in cases:
            Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for _, _, _, _, _, Y, eager in cases:
            assert torch.equal(Y, eager), rep
        # eager work between replays
        omq.w4a16_gemm(cases[0][0], cases[0][1], cases[0][2], cases[0][3], cases[0][4], 128)
        torch.cuda.synchronize()
