"""omq_lwc_backward_noalloc (the library's fixed device scratch, no workspace
argument) against omq_lwc_backward (caller workspace) through the C ABI: two calls
in a row on one GPU, the second on a smaller weight, each bit-identical to the
workspace form (the same kernels; every reduction runs in a fixed order), and the
first call's scratch contents must not leak into the second."""
import numpy as np
import pytest
import torch

import post_quantization_amd as omq
from oracle import quant
import synth
from gpu_util import dev, host, log

pytestmark = pytest.mark.gpu

F32 = np.float32


def _case(c_out, c_in, nbits, group, seed):
    rng = np.random.default_rng(seed)
    W = synth.normal(97, seed, (c_out, c_in), synth.WEIGHT_STD)
    rows = c_out * (c_in // group if group else 1)
    ag = rng.uniform(2.0, 5.0, rows).astype(F32)
    ab = rng.uniform(2.0, 5.0, rows).astype(F32)
    s = rng.uniform(0.7, 1.4, c_in).astype(F32)
    g = (rng.standard_normal((c_out, c_in)) * 1e-3).astype(F32)
    v = rng.standard_normal(c_out).astype(F32)
    tW = dev(W, torch.bfloat16)
    r = omq.lwc_fakequant(tW, dev(ag), dev(ab), nbits, dev(s), out_dtype=torch.bfloat16,
                          group=group)
    args = (dev(g), tW, nbits, dev(ag), dev(ab), r["h"], r["z"], r["arg_max"], r["arg_min"])
    kw = dict(s=dev(s), dy_colsum=dev(v), want_s=True, want_delta=True, group=group)
    return args, kw


def test_noalloc_matches_workspace_form_twice():
    assert omq.noalloc_scratch_bytes() == 64 << 20
    # the second call is smaller than the first
    for (c_out, c_in, nbits, group) in ((4096, 4096, 4, 0), (264, 640, 3, 128)):
        log("noalloc lwc_backward", c_out, c_in, nbits, group)
        args, kw = _case(c_out, c_in, nbits, group, c_out + c_in)
        want = omq.lwc_backward(*args, **kw)
        got = omq.lwc_backward_noalloc(*args, **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("g_a_gamma", "g_a_beta", "g_s", "g_delta"), got, want):
            a, b = host(a), host(b)
            assert np.isfinite(a).all(), name
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
