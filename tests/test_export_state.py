"""CPU checks of the export and driver helpers: the parameter-vector names follow the
library's packed layout (and the oracle's), and the saved calibration state and
exported tensors survive a save / load round trip, and the driver's starting
parameters are the oracle's."""
import numpy as np
import pytest
import torch

import post_quantization_amd as omq
from post_quantization_amd import export
from oracle import block as ob
import synth


@pytest.mark.parametrize("c", [synth.BLOCK_CFG4, synth.BLOCK_CFG5_W4, synth.FFN_CFG3_W2,
                               synth.BLOCK_CFG4_W3G128])
def test_theta_names_follow_the_layout(c):
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group)
    lay = ob.theta_layout(c, synth.block_weight_shapes(c))
    assert export.theta_names(d) == [n for n, _ in lay]
    theta = torch.arange(sum(k for _, k in lay), dtype=torch.float32)
    parts = export.theta_dict(d, theta)
    o = 0
    for n, k in lay:
        assert parts[n].numel() == k and int(parts[n][0]) == o
        o += k


def test_state_round_trip(tmp_path):
    c = synth.BLOCK_CFG4
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, lr_lwc=c.lr_lwc, lr_let=c.lr_let)
    rng = np.random.default_rng(0)
    th, m, v = (torch.from_numpy(rng.standard_normal(1000).astype(np.float32)) for _ in range(3))
    p = str(tmp_path / "state.safetensors")
    export.save_state(p, d, th, m, v, 17)
    th2, m2, v2, step, meta = export.load_state(p)
    assert step == 17 and meta["wbits"] == 4 and meta["d"] == 4096
    assert abs(meta["lr_let"] - 1e-2) < 1e-9
    for a, b in ((th, th2), (m, m2), (v, v2)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("c", [synth.BLOCK_CFG4, synth.BLOCK_CFG5_W2, synth.FFN_CFG3_W3,
                               synth.BLOCK_CFG4_W2G128])
def test_driver_initial_parameters(c):
    """The multi-block driver starts every block from the oracle's initial
    parameters (logits 4, s = 1, delta = 0, s_a = 1) in the packed layout."""
    from post_quantization_amd import driver
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group)
    shapes = synth.block_weight_shapes(c)
    want = ob.pack(c, shapes, ob.init_theta(c, shapes))
    assert np.array_equal(driver.init_theta(d, "cpu").numpy(), want)
