"""GPU parity of the block's causal attention (omq_attention_fwd / _bwd through the
C ABI) against the oracle's attention, element by element per head.

The attention of the quantized block (paper reading, section "LET": the affinity
of Q~ and K~, the softmax output kept in full precision) at the block workloads'
own sizes: T 2048 with 32 query heads on 32 KV heads (the 7B-shaped block: the
forward, the key-stationary dK/dV kernel and the query-stationary dQ kernel all run
their paired causal blocks) and with 64 query heads on 8 KV heads (the 70B-shaped
block: every kernel paired, the dK/dV kernel's query heads split four ways, with
the partial dK, dV added afterwards); plus a ragged paired case (T 2000), small
unpaired ones with ragged tails (the grouped ones with split query heads), and a
single query.

The oracle (float64) rounds P to bf16 for the P V product, as the kernel's operand
is (reading R20).  Inputs are bf16-exact, so the kernel's bf16 copy of dO is
lossless.  Tolerances: O and lse2 2e-3 relative per head (float32 softmax against
float64); dQ, dK, dV 2e-2 relative Frobenius per head (the kernel also rounds dS
to bf16 for its products, the bf16 path's tolerance).
"""
import numpy as np
import pytest
import torch

import post_quantization_amd as omq
from oracle import block as ob
from oracle import quant
import synth
from gpu_util import DEV, dev, host, log, rel

pytestmark = pytest.mark.gpu

HD = 128
CASES = {
    "mha32_t2048": (2048, 32, 32),
    "gqa64x8_t2048": (2048, 64, 8),
    "mha32_t2000_ragged": (2000, 32, 32),
    "gqa4x2_t1000_ragged": (1000, 4, 2),
    "mha2_t72": (72, 2, 2),
    "gqa2x1_t1": (1, 2, 1),
}


def _lse2(Q, K, n_q, n_kv, T):
    grp = n_q // n_kv
    out = np.zeros((n_q, T))
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    for h in range(n_q):
        g = h // grp
        S = Q[:, h * HD:(h + 1) * HD] @ K[:, g * HD:(g + 1) * HD].T / np.sqrt(HD)
        S[mask] = -np.inf
        mx = S.max(axis=1, keepdims=True)
        out[h] = (mx[:, 0] + np.log(np.exp(S - mx).sum(axis=1))) / np.log(2.0)
    return out


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind", list(CASES))
def test_attention_fwd_bwd(kind):
    T, n_q, n_kv = CASES[kind]
    log("attention", kind, "T", T, "n_q", n_q, "n_kv", n_kv)
    inp = synth.attention_inputs(9, T, n_q, n_kv)
    Q, K, V, dO = (inp[k].astype(np.float64) for k in ("Q", "K", "V", "dO"))
    O_ref, P = ob.attention(Q, K, V, n_q, n_kv, HD, cast=quant.bf16)
    dQ_ref, dK_ref, dV_ref = ob.attention_bwd(dO, Q, K, V, P, n_q, n_kv, HD)
    del P
    lse_ref = _lse2(Q, K, n_q, n_kv, T)

    tQ, tK, tV = (dev(inp[k], torch.bfloat16) for k in ("Q", "K", "V"))
    O, lse2 = omq.attention_fwd(tQ, tK, tV, n_q, n_kv)
    dQ, dK, dV = omq.attention_bwd(tQ, tK, tV, O, lse2, dev(inp["dO"]), n_q, n_kv)
    torch.cuda.synchronize()
    O, lse2, dQ, dK, dV = (host(t) for t in (O, lse2, dQ, dK, dV))
    assert np.isfinite(O).all() and np.isfinite(dQ).all()
    assert np.isfinite(dK).all() and np.isfinite(dV).all()
    worst = {}
    for h in range(n_q):
        sl = slice(h * HD, (h + 1) * HD)
        e_o = rel(O[:, sl], O_ref[:, sl])
        e_l = float(np.abs(lse2[h] - lse_ref[h]).max() / (1.0 + np.abs(lse_ref[h]).max()))
        e_q = rel(dQ[:, sl], dQ_ref[:, sl])
        for k, e in (("O", e_o), ("lse2", e_l), ("dQ", e_q)):
            worst[k] = max(worst.get(k, 0.0), e)
        assert e_o < 2e-3 and e_l < 2e-3, (h, e_o, e_l)
        assert e_q < 2e-2, (h, e_q)
    for g in range(n_kv):
        sl = slice(g * HD, (g + 1) * HD)
        e_k, e_v = rel(dK[:, sl], dK_ref[:, sl]), rel(dV[:, sl], dV_ref[:, sl])
        worst["dK"] = max(worst.get("dK", 0.0), e_k)
        worst["dV"] = max(worst.get("dV", 0.0), e_v)
        assert e_k < 2e-2 and e_v < 2e-2, (g, e_k, e_v)
    log("worst per head:", " ".join("%s %.2e" % kv for kv in worst.items()))
