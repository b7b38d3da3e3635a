"""Evaluation policy of the oracle forward passes.

TEST INFRASTRUCTURE ONLY (see the package header).

The linear and block forwards call the quantizer, the LET transforms and the
GEMM operand casts through an ``ops`` object.  ``ExactOps`` is the oracle
proper: the quantizer code path in exact float32 and, for the bf16 path, bf16
GEMM operands.  The tests plug in a float64 surrogate with frozen rounding /
clamping / argmax decisions to pin the hand-written backward by finite
differences.

Operand precision (``ExactOps(bf16=True)``, the bf16 path of reading R17): the
forward product of a layer whose weights and activations are both quantized is
the exact product of the dequantized values (``exact_product``); every other
matrix product -- a weight-only layer's forward, every backward product, and
the attention products -- takes its operands rounded to bf16 as the matrix
cores take them, with float64 accumulation.
"""
from __future__ import annotations

import numpy as np

from . import quant

F32 = np.float32
F64 = np.float64


class ExactOps:
    # the RMSNorm rows entering a quantizer take the code path's rounding (R29)
    rms_rounding = True

    def __init__(self, bf16: bool):
        self.bf16 = bf16
        self.states = {}

    # gamma / beta from their logits
    def sigmoid(self, a):
        return quant.sigmoid32(a)

    def to_code(self, x):
        """Entry into the float32 code path."""
        return np.asarray(x, dtype=F64).astype(F32)

    def let_act(self, X, s, delta):
        return quant.let_act(self.to_code(X), s, delta)

    def let_weight(self, W, s):
        return quant.let_weight(W, s)

    def div(self, X, s):
        """Q~ = Q / s_a (the LET of the attention affinity on the query side)."""
        return self.to_code(X) / np.asarray(s, dtype=F32)[None, :]

    def mul(self, X, s):
        """K~ = s_a * K (the key side)."""
        return np.asarray(s, dtype=F32)[None, :] * self.to_code(X)

    def quant(self, x, gamma, beta, nbits, key):
        st = quant.quantize_rows(self.to_code(x), gamma, beta, nbits)
        self.states[key] = st
        return st

    def act(self, x, abits, key):
        if abits >= 16:
            return None, self.to_code(x)
        st = self.quant(x, F32(1), F32(1), abits, key)
        return st, st.xhat

    def operand(self, a):
        """A GEMM operand as the GPU feeds it to the matrix cores."""
        if self.bf16:
            return quant.bf16(a)
        return np.asarray(a, dtype=F64)

    def grad_operand(self, g):
        """An upstream gradient as a backward product takes it (dL/dY of a linear
        layer, dL/dO and dL/dS of the attention): in bf16 on the bf16 path, like
        every other matrix-core operand (reading R17)."""
        return self.operand(g)

    def prob(self, P):
        """The softmax output as the P V product takes it: the bf16 path feeds the
        normalized probabilities to the matrix cores rounded to bf16 (reading R20);
        the softmax itself is never quantized."""
        return self.operand(P)

    def exact_product(self, wbits, abits):
        """Whether a linear layer's forward product takes the exact quantized operands.

        The method's quantized layer computes Y = Q_a(X~) Q_w(W~) + B~ (paper reading,
        section "LET"), each quantized operand being (q - z) h per quantizer row
        (section "LWC").  When both quantizers are on, that product is formed from
        the exact dequantized values (float32, products and sums in float64): the
        definition written out, whatever the widths, bit widths or LWC grouping.
        When one side is unquantized its operand is a plain float tensor, which the
        bf16 path feeds to the matrix cores in bf16 (reading R17), so the product
        takes the operand() casts.  The backward's products always take operand()."""
        return wbits < 16 and abits < 16
