"""Sequential multi-block calibration of a stack of decoder blocks.

Paper reading ("OmniQuant: ...", section "框架", the block-wise objective and the
flowchart after it; section "实验证据" for the schedule): blocks are calibrated one
after another; block k's objective compares the full-precision block F(W, X) with
the quantized block on the same input X; once block k is calibrated and frozen,
its quantized output is block k+1's input.  The schedule is batch size 1, a fixed
number of epochs over the calibration samples, AdamW with separate learning rates
for the clipping logits and the LET parameters.

Per block, with x_i the samples' current inputs (bf16, resident in HBM):
  1. targets y*_i = F(W, x_i) with the raw weights, cached in fp32 for every sample;
  2. epochs x samples calibration steps (quantized forward on x_i, MSE against y*_i,
     straight-through backward, AdamW), the step count restarting at 1 per block;
  3. x_i <- bf16(F_q(W; Theta)(x_i)), the next block's inputs.
Every step runs in the library's kernels (block forward / step); this module only
orders the calls.  A block whose parameters are given (resume) skips 1-2 and only
advances the inputs.
"""
from __future__ import annotations

import time
from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence

import torch

from . import BlockDesc, block_forward, block_step, block_theta_layout, block_workspace_size
from .export import theta_names


def init_theta(desc: BlockDesc, device, a0: float = 4.0) -> torch.Tensor:
    """The packed parameters at the start of a block: clipping logits a0 (so
    gamma = beta = sigmoid(a0)), LET scales 1, shifts 0, s_a 1."""
    offs, _, total = block_theta_layout(desc)
    ends = list(offs[1:]) + [total]
    th = torch.empty(total, dtype=torch.float32, device=device)
    for name, a, b in zip(theta_names(desc), offs, ends):
        th[a:b] = a0 if name.startswith("a_") else (0.0 if name.startswith("delta_") else 1.0)
    return th


@dataclass
class StepState:
    """What a step hook sees (device tensors, valid until the next step)."""
    block: int
    epoch: int
    sample: int
    step: int
    theta: torch.Tensor
    dtheta: torch.Tensor
    adam_m: torch.Tensor
    adam_v: torch.Tensor
    loss: torch.Tensor


@dataclass
class CalibResult:
    thetas: List[torch.Tensor]
    outputs: torch.Tensor            # [n, T, d] bf16: the last block's quantized outputs
    seconds: List[float]             # wall time per block (targets + steps + next inputs)


def calibrate(desc: BlockDesc, blocks: Sequence[Sequence[Optional[torch.Tensor]]],
              samples: torch.Tensor, epochs: int, a0: float = 4.0,
              done: Sequence[torch.Tensor] = (),
              on_step: Optional[Callable[[StepState], None]] = None,
              on_block: Optional[Callable[[int, torch.Tensor, torch.Tensor], None]] = None
              ) -> CalibResult:
    """desc: the block shape and optimizer setup (T = tokens per sample);
    blocks: per block the 7 bf16 [C_out x C_in] weights (q, k, v, o, gate, up, down;
    None for the attention ones of an FFN-only stack); samples: bf16 [n, T, d] on the
    device (not modified); done: calibrated parameters of the leading blocks (resume);
    on_step(state) after every step (reading state tensors synchronizes);
    on_block(b, inputs, theta) once block b is calibrated, with its inputs."""
    if samples.dim() != 3 or samples.shape[1] != desc.T or samples.shape[2] != desc.d:
        raise ValueError("samples must be [n, T, d]")
    if samples.dtype != torch.bfloat16:
        raise ValueError("samples must be bf16")
    dev = samples.device
    n = samples.shape[0]
    ws = torch.empty(block_workspace_size(desc), dtype=torch.uint8, device=dev)
    x = samples.clone()
    y_t = torch.empty(n, desc.T, desc.d, dtype=torch.float32, device=dev)
    y = torch.empty(desc.T, desc.d, dtype=torch.float32, device=dev)
    loss = torch.zeros(1, dtype=torch.float32, device=dev)
    res = CalibResult([], x, [])
    for b, W in enumerate(blocks):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if b < len(done):
            theta = done[b].to(dev, torch.float32).contiguous()
        else:
            for i in range(n):
                block_forward(desc, x[i], W, None, y_t[i], ws)
            theta = init_theta(desc, dev, a0)
            dtheta = torch.zeros_like(theta)
            m = torch.zeros_like(theta)
            v = torch.zeros_like(theta)
            step = 0
            for e in range(epochs):
                for i in range(n):
                    step += 1
                    block_step(desc, x[i], y_t[i], W, theta, dtheta, m, v, step, loss, ws)
                    if on_step is not None:
                        on_step(StepState(b, e, i, step, theta, dtheta, m, v, loss))
        if on_block is not None:
            on_block(b, x, theta)
        for i in range(n):
            block_forward(desc, x[i], W, theta, y, ws)
            x[i].copy_(y)
        torch.cuda.synchronize()
        res.thetas.append(theta)
        res.seconds.append(time.perf_counter() - t0)
    return res
