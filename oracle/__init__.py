"""CPU oracle of OmniQuant's block-wise calibration step (LWC + LET, STE backward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The GPU library never routes through it, and it imports nothing from the GPU
path (``post_quantization_amd``); the two share no code.  Seeded inputs come
from the separate ``synth`` module, which holds none of the method's arithmetic.

Source of truth: the paper reading "OmniQuant: Omnidirectionally Calibrated
Quantization for Large Language Models" (onecrewdev.com/posts/omniquant-paper-reading):
its block-wise objective (section "框架"), the LWC equation (section "LWC"), the LET
equations for linear layers and for the attention affinity (section "LET"), and the
experimental setup (section "实验证据").  The affine worked example of the
quantization tutorial (devpress.csdn.net, section 2.2) pins the quantizer.

Precision: the quantizer code path (clipping range, step size h, zero point z,
integer codes, dequantized values, and the LET divisions feeding it) is evaluated
exactly in float32, one IEEE operation at a time (numpy float32 ufuncs, np.rint
= round half to even, true division, no fused multiply-add).  Everything else
(GEMMs, attention, norms, reductions, gradients) runs in float64.  For the bf16
path the operands of every GEMM that the GPU runs in bf16 (dequantized weights
and activations, attention Q/K/V) are rounded to bf16 (nearest-even) before a
float64 product.

Parity status of each function is stated in its module header; every function
here is pinned by a CPU test (tests/test_oracle_*.py).
"""
from . import quant, linear, block, optim  # noqa: F401
