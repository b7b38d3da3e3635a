"""Evaluation policy of the oracle forward passes.

TEST INFRASTRUCTURE ONLY (see the package header).

The linear and block forwards call the quantizer, the LET transforms and the
GEMM operand casts through an ``ops`` object.  ``ExactOps`` is the oracle
proper: the quantizer code path in exact float32 and, for the bf16 path, bf16
GEMM operands.  The tests plug in a float64 surrogate with frozen rounding /
clamping / argmax decisions to pin the hand-written backward by finite
differences.
"""
from __future__ import annotations

import numpy as np

from . import quant

F32 = np.float32
F64 = np.float64


class ExactOps:
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

    def code_product(self, c):
        """Whether the bf16 path forms the block forward's four quantized products
        (quantized activations times LWC weights) on the integer codes: exactly
        (q_x - z_x) h_x times (q_w - z_w) h_w, no operand rounding.  It does so for
        per-row quantizers with codes below 128 on both sides and every input width
        a multiple of 16; otherwise the operands enter as bf16 like any other.  The
        backward's products take the bf16 operands either way."""
        widths = [c.d, c.F] + ([] if c.ffn_only else [c.n_q * c.head_dim])
        return (self.bf16 and c.wbits <= 7 and c.abits <= 7 and not c.group
                and all(w % 16 == 0 for w in widths))
