"""Seeded synthetic workloads for the OmniQuant block-calibration path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the quantization method: only the shapes
of the workloads, seeded random draws, and rounding of those draws to the
storage type (bf16) they are handed over in.

Every tensor comes from ``numpy.random.default_rng([cfg, tensor_id])`` (PCG64),
drawn in float32.  bf16 tensors are the float32 draws rounded to nearest-even
bf16 and returned as float32 arrays whose values are exactly representable in
bf16 (``bf16_bits`` gives the 16-bit patterns to upload).

The calibration data of the method (128 random 2048-token WikiText2 segments of
real LLaMA activations, per the paper reading's experimental setup) and LLaMA
weights are not available; these inputs stand in for them with the same token
count and hidden sizes, and with the systematic outlier channels the paper
reading describes for LLM activations (a few fixed channels scaled up).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np

WEIGHT_STD = 0.02


def rng(cfg: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(cfg), int(tensor_id)])


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """16-bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def normal(cfg: int, tid: int, shape, std: float = 1.0, bf16: bool = True) -> np.ndarray:
    a = rng(cfg, tid).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16(a) if bf16 else a


def outlier_activations(cfg: int, tid: int, T: int, C: int, n_out: int,
                        lo: float, hi: float, bf16: bool = True,
                        channels: Optional[Tuple[int, ...]] = None) -> np.ndarray:
    """X ~ N(0,1) [T x C] with ``n_out`` seeded channels (columns) scaled by
    U(lo, hi) (a fixed factor when lo == hi), re-rounded to bf16."""
    x = normal(cfg, tid, (T, C), 1.0, bf16=bf16)
    g = rng(cfg, tid + 1000)
    if channels is None:
        ch = g.choice(C, size=n_out, replace=False)
    else:
        ch = np.asarray(channels, dtype=np.int64)
    if lo == hi:
        fac = np.full(len(ch), lo, dtype=np.float32)
    else:
        fac = g.uniform(lo, hi, size=len(ch)).astype(np.float32)
    x[:, ch] *= fac[None, :]
    return to_bf16(x) if bf16 else x


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class LinearCfg:
    """One quantized linear layer: Y = X W^T + B, W is [c_out x c_in]."""
    cfg: int
    T: int
    c_in: int
    c_out: int
    wbits: int
    abits: int
    let: bool
    fp32: bool                 # fp32 storage / fp32 GEMM path
    n_out: int                 # outlier channel count
    out_lo: float
    out_hi: float
    out_channels: Optional[Tuple[int, ...]] = None
    steps: int = 1
    opt: str = "adamw"         # "sgd" or "adamw"
    lr_lwc: float = 5e-3
    lr_let: float = 1e-2


@dataclass(frozen=True)
class BlockCfg:
    """A LLaMA-shaped decoder block (or its FFN alone when ffn_only)."""
    cfg: int
    T: int
    d: int
    n_q: int
    n_kv: int
    F: int
    wbits: int
    abits: int
    head_dim: int = 128
    ffn_only: bool = False
    n_out: int = 41
    out_lo: float = 20.0
    out_hi: float = 100.0
    steps: int = 20
    lr_lwc: float = 5e-3
    lr_let: float = 1e-2
    rope_theta: float = 10000.0
    eps: float = 1e-6
    group: int = 0             # LWC group size along C_in; 0: one group per output channel


LINEAR_CFG1 = LinearCfg(cfg=1, T=16, c_in=64, c_out=32, wbits=4, abits=16, let=False,
                        fp32=True, n_out=2, out_lo=50.0, out_hi=50.0, out_channels=(3, 17),
                        steps=10, opt="sgd")
LINEAR_CFG2 = LinearCfg(cfg=2, T=2048, c_in=4096, c_out=4096, wbits=4, abits=4, let=True,
                        fp32=False, n_out=41, out_lo=20.0, out_hi=100.0)
FFN_CFG3_W3 = BlockCfg(cfg=3, T=2048, d=4096, n_q=32, n_kv=32, F=11008, wbits=3, abits=16,
                       ffn_only=True, n_out=41, out_lo=50.0, out_hi=50.0)
FFN_CFG3_W2 = replace(FFN_CFG3_W3, wbits=2)
BLOCK_CFG4 = BlockCfg(cfg=4, T=2048, d=4096, n_q=32, n_kv=32, F=11008, wbits=4, abits=4)
BLOCK_CFG5_W4 = BlockCfg(cfg=5, T=2048, d=8192, n_q=64, n_kv=8, F=28672, wbits=4, abits=16,
                         n_out=82)
BLOCK_CFG5_W2 = replace(BLOCK_CFG5_W4, wbits=2)
# group-wise LWC (128 input channels per clipping group), weight-only: the pages'
# headline W3A16g128 / W2A16g128 settings on the 7B-shaped block
BLOCK_CFG4_W3G128 = replace(BLOCK_CFG4, wbits=3, abits=16, group=128)
BLOCK_CFG4_W2G128 = replace(BLOCK_CFG4, wbits=2, abits=16, group=128)


def linear_inputs(c: LinearCfg) -> Dict[str, np.ndarray]:
    bf = not c.fp32
    W = normal(c.cfg, 1, (c.c_out, c.c_in), WEIGHT_STD, bf16=bf)
    X = outlier_activations(c.cfg, 2, c.T, c.c_in, c.n_out, c.out_lo, c.out_hi, bf16=bf,
                            channels=c.out_channels)
    B = np.zeros(c.c_out, dtype=np.float32)
    return {"W": W, "X": X, "B": B}


WEIGHT_NAMES = ("q", "k", "v", "o", "gate", "up", "down")


def block_weight_shapes(c: BlockCfg) -> Dict[str, Tuple[int, int]]:
    dq = c.n_q * c.head_dim
    dk = c.n_kv * c.head_dim
    return {"q": (dq, c.d), "k": (dk, c.d), "v": (dk, c.d), "o": (c.d, dq),
            "gate": (c.F, c.d), "up": (c.F, c.d), "down": (c.d, c.F)}


def block_inputs(c: BlockCfg) -> Dict[str, np.ndarray]:
    out: Dict[str, np.ndarray] = {}
    shapes = block_weight_shapes(c)
    names = ("gate", "up", "down") if c.ffn_only else WEIGHT_NAMES
    for i, n in enumerate(WEIGHT_NAMES):
        if n in names:
            out["W_" + n] = normal(c.cfg, 10 + i, shapes[n], WEIGHT_STD, bf16=True)
    out["x"] = outlier_activations(c.cfg, 2, c.T, c.d, c.n_out, c.out_lo, c.out_hi, bf16=True)
    return out


def stack_inputs(c: BlockCfg, n_blocks: int, n_samples: int):
    """A stack of n_blocks blocks and n_samples calibration samples.

    Block b's weights use tensor ids 100 b + 10 + i (block 0 is block_inputs'
    weights); sample s is an outlier-activation draw with tensor id 100000 + s and
    its factors from id 101000 + s, on the same outlier channels for every sample
    (the channels block_inputs picks).  Returns (list of weight dicts, samples
    float32 [n_samples, T, d] with bf16-exact values)."""
    assert n_samples <= 1000 and n_blocks <= 900
    shapes = block_weight_shapes(c)
    names = ("gate", "up", "down") if c.ffn_only else WEIGHT_NAMES
    blocks = []
    for b in range(n_blocks):
        blocks.append({"W_" + n: normal(c.cfg, 100 * b + 10 + i, shapes[n], WEIGHT_STD)
                       for i, n in enumerate(WEIGHT_NAMES) if n in names})
    ch = tuple(int(v) for v in rng(c.cfg, 1002).choice(c.d, size=c.n_out, replace=False))
    xs = np.empty((n_samples, c.T, c.d), dtype=np.float32)
    for s in range(n_samples):
        xs[s] = outlier_activations(c.cfg, 100000 + s, c.T, c.d, c.n_out, c.out_lo, c.out_hi,
                                    channels=ch)
    return blocks, xs


def stack_samples_device(c: BlockCfg, n_samples: int, device, seed: int = 0):
    """n_samples calibration samples [n, T, d] bf16 drawn on the device (for the
    full-size throughput runs, where the numpy draws of stack_inputs take minutes):
    the same recipe (N(0, 1), the block_inputs outlier channels scaled by U(lo, hi)
    per sample) from torch's seeded generator; not the values stack_inputs gives."""
    import torch
    ch = torch.as_tensor(rng(c.cfg, 1002).choice(c.d, size=c.n_out, replace=False),
                         device=device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(c.cfg))
    x = torch.randn(n_samples, c.T, c.d, generator=g, device=device, dtype=torch.float32)
    fac = torch.rand(n_samples, 1, c.n_out, generator=g, device=device) * (c.out_hi - c.out_lo)
    x[:, :, ch] *= fac + c.out_lo
    return x.to(torch.bfloat16)


def reduced(c, **kw):
    """The same workload at other sizes (parity cases the oracle finishes fast)."""
    return replace(c, **kw)


def attention_inputs(cfg: int, T: int, n_q: int, n_kv: int, hd: int = 128,
                     q_scale: float = 2.0) -> Dict[str, np.ndarray]:
    """bf16 Q [T x n_q hd], K, V [T x n_kv hd] ~ N(0, 1) (Q times q_scale, for a
    softmax with some sharp rows) and an upstream gradient dO [T x n_q hd] ~ N(0, 1),
    all bf16-exact float32 arrays (tensor ids 20-23 of workload cfg)."""
    return {"Q": to_bf16(normal(cfg, 20, (T, n_q * hd), bf16=False) * np.float32(q_scale)),
            "K": normal(cfg, 21, (T, n_kv * hd)),
            "V": normal(cfg, 22, (T, n_kv * hd)),
            "dO": normal(cfg, 23, (T, n_q * hd))}
