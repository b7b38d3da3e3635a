"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/omq.h declares, rejects bad arguments before launching anything, and its
host-side layouts (packed theta, workspace sizes) agree with the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import post_quantization_amd as omq
from oracle import block as ob
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "omq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(omq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    L = omq.lib()
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert omq.abi_version() == 4


def test_status_strings():
    assert omq.status_str(0) == "ok"
    for rc in range(-1, -8, -1):
        assert omq.status_str(rc) not in ("ok", "unknown status")
    assert omq.status_str(-99) == "unknown status"


FAKE = 0x10000  # a 16-byte aligned non-NULL address; never dereferenced (validation fails first)


def test_validation_before_launch():
    L = omq.lib()
    # missing required pointer
    assert L.omq_lwc_fakequant(None, 1, 4, 8, 0, 4, FAKE, FAKE, None, None, None, FAKE, 1, FAKE,
                               FAKE, FAKE, FAKE, None, None, None, None) == -1
    # bit width out of range
    assert L.omq_lwc_fakequant(FAKE, 1, 4, 8, 0, 9, FAKE, FAKE, None, None, None, FAKE, 1, FAKE,
                               FAKE, FAKE, FAKE, None, None, None, None) == -1
    assert L.omq_act_quant(FAKE, 1, 4, 8, 1, 0, None, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                           None, None, None) == -1
    # bad dtype
    assert L.omq_act_quant(FAKE, 7, 4, 8, 4, 0, None, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                           None, None, None) == -3
    # LET mode without s
    assert L.omq_act_quant(FAKE, 1, 4, 8, 4, 1, None, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                           None, None, None) == -1
    # row length not a multiple of 4
    assert L.omq_act_quant(FAKE, 1, 4, 10, 4, 0, None, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                           None, None, None) == -4
    # misaligned input-health flag
    assert L.omq_act_quant(FAKE, 1, 4, 8, 4, 0, None, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                           None, FAKE + 2, None) == -4
    # misaligned pointer
    assert L.omq_act_quant(FAKE + 2, 1, 4, 8, 4, 0, None, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                           None, None, None) == -4
    # bf16 GEMM needs K % 8 == 0
    assert L.omq_gemm(4, 4, 12, FAKE, 12, 0, FAKE, 12, 0, 1, None, 1.0, FAKE, 4, 0, None) == -4
    assert L.omq_gemm(4, 4, 16, FAKE, 8, 0, FAKE, 16, 0, 1, None, 1.0, FAKE, 4, 0, None) == -2
    # transposed A: its contiguous extent is M (here 12, not a multiple of 8)
    assert L.omq_gemm(12, 8, 16, FAKE, 12, 1, FAKE, 16, 0, 1, None, 1.0, FAKE, 8, 0, None) == -4
    # integer-code product: K, lda, ldb multiples of 16, 16-byte aligned codes, K <= 2^17
    assert L.omq_code_gemm(4, 4, 24, FAKE, 24, FAKE, FAKE, FAKE, FAKE, 24, FAKE, FAKE, FAKE,
                           None, FAKE, 4, None) == -4
    assert L.omq_code_gemm(4, 4, 32, FAKE + 8, 32, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE,
                           None, FAKE, 4, None) == -4
    assert L.omq_code_gemm(4, 4, 32, FAKE, 32, FAKE, FAKE, None, FAKE, 32, FAKE, FAKE, FAKE,
                           None, FAKE, 4, None) == -1
    assert L.omq_code_gemm(4, 4, 1 << 18, FAKE, 1 << 18, FAKE, FAKE, FAKE, FAKE, 1 << 18, FAKE,
                           FAKE, FAKE, None, FAKE, 4, None) == -2
    assert L.omq_code_rowsum(FAKE, 4, 32, 16, FAKE, None) == -2
    # unsupported LWC group (only per channel or 128 input channels)
    assert L.omq_lwc_fakequant(FAKE, 1, 4, 256, 64, 4, FAKE, FAKE, None, None, None, FAKE, 1,
                               FAKE, FAKE, FAKE, FAKE, None, None, None, None) == -2
    assert L.omq_lwc_fakequant(FAKE, 1, 4, 200, 128, 4, FAKE, FAKE, None, None, None, FAKE, 1,
                               FAKE, FAKE, FAKE, FAKE, None, None, None, None) == -2
    # workspace too small
    assert L.omq_lwc_backward(FAKE, FAKE, 1, 8, 8, 0, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                              None, FAKE, FAKE, None, None, FAKE, 16, None) == -5
    # the fixed-scratch form: shapes whose partials exceed the array are refused
    assert omq.noalloc_scratch_bytes() == 64 << 20
    assert L.omq_lwc_backward_noalloc(FAKE, FAKE, 1, 28672, 8192, 0, 4, FAKE, FAKE, None, FAKE,
                                      FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, None) == -5
    assert L.omq_lwc_backward_noalloc(FAKE, FAKE, 1, 8, 0, 0, 4, FAKE, FAKE, None, FAKE, FAKE,
                                      FAKE, FAKE, None, FAKE, FAKE, None, None, None) == -2
    assert L.omq_adamw(FAKE, FAKE, FAKE, FAKE, 10, 4, 1e-3, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0,
                       None) == -1
    d = omq.QLinearDesc(T=12, c_in=16, c_out=8, wbits=4, abits=4, use_let=1, path=omq.PATH_BF16)
    assert omq.qlinear_workspace_size(d) == 0          # bf16 path needs T % 8 == 0
    d = omq.QLinearDesc(T=16, c_in=16, c_out=8, wbits=4, abits=4, use_let=1, path=omq.PATH_BF16)
    assert omq.qlinear_workspace_size(d) > 0
    assert L.omq_qlinear_fwd(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, 64, None) == -5
    b = omq.BlockDesc(T=64, d=64, n_q=3, n_kv=2, head_dim=16, F=64, wbits=4, abits=4)
    assert omq.block_workspace_size(b) == 0            # n_q not a multiple of n_kv
    b = omq.BlockDesc(T=64, d=256, n_q=4, n_kv=4, head_dim=64, F=64, wbits=4, abits=4)
    assert omq.block_workspace_size(b) == 0            # the attention kernels take head_dim 128
    b = omq.BlockDesc(T=64, d=256, n_q=2, n_kv=2, head_dim=128, F=64, wbits=4, abits=4)
    assert omq.block_workspace_size(b) > 0
    # group-wise clipping with quantized activations: not implemented
    b = omq.BlockDesc(T=64, d=256, n_q=2, n_kv=2, head_dim=128, F=256, wbits=4, abits=4,
                      group=128)
    assert omq.block_workspace_size(b) == 0
    assert L.omq_block_theta_layout(ctypes.byref(b), None, None, None, None) == -7
    b = omq.BlockDesc(T=64, d=256, n_q=2, n_kv=2, head_dim=128, F=256, wbits=4, abits=16,
                      group=128)
    assert omq.block_workspace_size(b) > 0
    # 8-bit codes and widths that are not multiples of 16 run the exact code product
    b = omq.BlockDesc(T=64, d=264, n_q=2, n_kv=2, head_dim=128, F=200, wbits=8, abits=8)
    assert omq.block_workspace_size(b) > 0
    # attention on quantized operands: head_dim 128 only, strides and alignment
    assert L.omq_attention_fwd(FAKE, 512, FAKE, FAKE, 256, 64, 4, 2, 64, FAKE, 512, FAKE,
                               None) == -2
    assert L.omq_attention_fwd(FAKE, 512, FAKE, FAKE, 256, 64, 4, 3, 128, FAKE, 512, FAKE,
                               None) == -2
    assert L.omq_attention_fwd(FAKE, 500, FAKE, FAKE, 256, 64, 4, 2, 128, FAKE, 512, FAKE,
                               None) == -2
    assert L.omq_attention_fwd(FAKE, 516, FAKE, FAKE, 256, 64, 4, 2, 128, FAKE, 512, FAKE,
                               None) == -4
    assert L.omq_attention_fwd(FAKE, 512, FAKE, FAKE, 256, 64, 4, 2, 128, FAKE, 512, None,
                               None) == -1
    assert L.omq_attention_fwd(FAKE, 512, FAKE, FAKE, 256, 0, 4, 2, 128, FAKE, 512, FAKE,
                               None) == 0
    assert L.omq_attention_bwd(FAKE, 512, FAKE, FAKE, 256, 64, 4, 2, 128, FAKE, FAKE, 512, FAKE,
                               FAKE, 512, FAKE, FAKE, 256, FAKE, 16, None) == -5
    assert omq.lib().omq_attention_bwd_workspace_size(64, 4, 512) >= 64 * 4 * 4 + 64 * 512 * 2
    # grouped K/V heads too few to fill the device: the dK/dV pass splits a group's query
    # heads and keeps float32 partial dK, dV of all splits but the first; the size covers
    # the largest need over every n_kv dividing n_q (64 query heads at 2048 tokens: one
    # K/V head, 8 paired key blocks, 32 splits); then the bf16 dS of every head,
    # [2048 keys x 2048 queries] each
    need = (64 * 2048 * 4 + 2048 * 8192 * 2 + 31 * 2 * 2048 * 1 * 128 * 4
            + 64 * 2048 * 2048 * 2)
    assert omq.lib().omq_attention_bwd_workspace_size(2048, 64, 8192) >= need
    assert omq.lib().omq_attention_bwd_workspace_size(2048, 64, 8192) < need + 4096
    # a dS scratch beyond 2^50 elements: no size, and the call is refused as a shape error
    assert omq.lib().omq_attention_bwd_workspace_size(1 << 26, 4, 512) == 0
    assert L.omq_attention_bwd(FAKE, 512, FAKE, FAKE, 256, 1 << 26, 4, 2, 128, FAKE, FAKE, 512,
                               FAKE, FAKE, 512, FAKE, FAKE, 256, FAKE, 1 << 62, None) == -2
    b = omq.BlockDesc(T=64, d=64, n_q=4, n_kv=2, head_dim=16, F=64, wbits=4, abits=4,
                      optimizer=5)
    assert L.omq_block_step(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None,
                            FAKE, 1 << 30, None) == -1


@pytest.mark.parametrize("kind", ["mha_w4a4", "gqa_w4a16", "ffn_w2a16", "mha_w3a16g128"])
def test_block_theta_layout_matches_oracle(kind):
    c = {"mha_w4a4": synth.BLOCK_CFG4, "gqa_w4a16": synth.BLOCK_CFG5_W4,
         "ffn_w2a16": synth.FFN_CFG3_W2, "mha_w3a16g128": synth.BLOCK_CFG4_W3G128}[kind]
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group)
    offs, n_lwc, total = omq.block_theta_layout(d)
    lay = ob.theta_layout(c, synth.block_weight_shapes(c))
    sizes = [n for _, n in lay]
    assert total == sum(sizes)
    assert offs == list(np.cumsum([0] + sizes[:-1]))
    assert n_lwc == sum(n for name, n in lay if name.startswith("a_"))
    assert omq.block_workspace_size(d) > 0


def test_empty_outputs_return_ok_without_touching_pointers():
    """Calls whose outputs have no rows return OMQ_OK before any pointer is read, so
    they run here, where there is no GPU (NULL pointers: nothing is dereferenced)."""
    L = omq.lib()
    assert L.omq_act_quant(None, 1, 0, 8, 4, 0, None, None, None, 1, None, None, None, None,
                           None, None, None) == 0
    assert L.omq_lwc_fakequant(None, 1, 0, 8, 0, 4, None, None, None, None, None, None, 1,
                               None, None, None, None, None, None, None, None) == 0
    assert L.omq_gemm(0, 4, 16, None, 16, 0, None, 16, 0, 1, None, 1.0, None, 4, 0, None) == 0
    assert L.omq_gemm(4, 0, 16, None, 16, 0, None, 16, 0, 1, None, 1.0, None, 0, 0, None) == 0
    assert L.omq_code_gemm(0, 4, 16, None, 16, None, None, None, None, 16, None, None, None,
                           None, None, 4, None) == 0
    # negative sizes stay errors
    assert L.omq_act_quant(None, 1, -1, 8, 4, 0, None, None, None, 1, None, None, None, None,
                           None, None, None) != 0
