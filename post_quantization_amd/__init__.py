"""Python binding of libomq (OmniQuant block calibration on MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/omq.h.  PyTorch provides device memory and the current
stream.  Importing this package without the built library raises (build with
``python -m post_quantization_amd.build``); there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

__all__ = [
    "OmqError", "lib", "status_str", "abi_version", "lwc_fakequant", "let_apply", "act_quant",
    "gemm", "lwc_backward", "act_quant_backward", "QLinearDesc", "qlinear_theta_size",
    "qlinear_workspace_size", "qlinear_fwd", "qlinear_bwd", "sgd", "adamw", "BlockDesc",
    "block_theta_layout", "block_workspace_size", "block_forward", "block_step",
    "F32", "BF16", "LET_NONE", "LET_DIV", "LET_MUL", "PATH_FP32", "PATH_BF16",
    "OPT_ADAMW", "OPT_SGD", "GemmTimer", "pack_codes", "fold_linear", "w4a16_gemm",
    "attention_fwd", "attention_bwd", "lwc_backward_noalloc", "noalloc_scratch_bytes",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libomq.so")

F32, BF16 = 0, 1
LET_NONE, LET_DIV, LET_MUL = 0, 1, 2
PATH_FP32, PATH_BF16 = 0, 1
OPT_ADAMW, OPT_SGD = 0, 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p
_f = ctypes.c_float
_sz = ctypes.c_size_t


class OmqError(RuntimeError):
    pass


class QLinearDesc(ctypes.Structure):
    _fields_ = [("struct_size", _sz), ("T", _i64), ("c_in", _i64), ("c_out", _i64),
                ("wbits", _int), ("abits", _int), ("use_let", _int), ("path", _int),
                ("group", _i64)]

    def __init__(self, T, c_in, c_out, wbits, abits, use_let, path, group=0):
        super().__init__(ctypes.sizeof(QLinearDesc), T, c_in, c_out, wbits, abits,
                         int(use_let), path, group)


TIMED_GEMM, TIMED_GEMM_I8, TIMED_WEIGHT_QUANT, TIMED_ACT_QUANT = 0, 1, 2, 3


class OmqTimer(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("capacity", _int),
                ("count", _int), ("flops", ctypes.c_double),
                ("kinds", ctypes.POINTER(ctypes.c_int)), ("flops_codes", ctypes.c_double),
                ("work", ctypes.POINTER(ctypes.c_double))]


def _hip():
    """The HIP runtime already loaded in this process (torch's)."""
    path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    return ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")


class GemmTimer:
    """Event pairs the library records around each matrix-core GEMM of a block step."""

    def __init__(self, capacity: int):
        hip = _hip()
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        self._hip = hip
        self._ev = (ctypes.c_void_p * (2 * capacity))()
        for i in range(2 * capacity):
            e = ctypes.c_void_p()
            rc = hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise OmqError("hipEventCreate failed (%d)" % rc)
            self._ev[i] = e.value
        self._kinds = (ctypes.c_int * capacity)()
        self._work = (ctypes.c_double * capacity)()
        self.struct = OmqTimer(ctypes.cast(self._ev, ctypes.POINTER(ctypes.c_void_p)), capacity,
                               0, 0.0, ctypes.cast(self._kinds, ctypes.POINTER(ctypes.c_int)),
                               0.0, ctypes.cast(self._work, ctypes.POINTER(ctypes.c_double)))

    def reset(self):
        self.struct.count = 0
        self.struct.flops = 0.0
        self.struct.flops_codes = 0.0

    def kinds(self):
        """Per recorded launch: TIMED_GEMM, TIMED_GEMM_I8, TIMED_WEIGHT_QUANT or
        TIMED_ACT_QUANT."""
        return [self._kinds[i] for i in range(self.struct.count)]

    def work(self):
        """Per recorded launch: algorithmic FLOPs (GEMMs) or HBM bytes (quantizers)."""
        return [self._work[i] for i in range(self.struct.count)]

    def durations_ms(self):
        out = []
        f = ctypes.c_float()
        for i in range(self.struct.count):
            rc = self._hip.hipEventElapsedTime(ctypes.byref(f), self._ev[2 * i],
                                               self._ev[2 * i + 1])
            if rc != 0:
                raise OmqError("hipEventElapsedTime failed (%d)" % rc)
            out.append(f.value)
        return out


class BlockDesc(ctypes.Structure):
    _fields_ = [("struct_size", _sz), ("T", _i64), ("d", _i64), ("n_q", _i64),
                ("n_kv", _i64), ("head_dim", _i64), ("F", _i64), ("wbits", _int),
                ("abits", _int), ("ffn_only", _int), ("eps", _f), ("rope_theta", _f),
                ("optimizer", _int), ("lr_lwc", _f), ("lr_let", _f), ("beta1", _f),
                ("beta2", _f), ("adam_eps", _f), ("weight_decay", _f),
                ("timer", ctypes.POINTER(OmqTimer)), ("group", _i64), ("nonfinite", _vp)]

    def __init__(self, T, d, n_q, n_kv, head_dim, F, wbits, abits, ffn_only=False, eps=1e-6,
                 rope_theta=10000.0, optimizer=OPT_ADAMW, lr_lwc=5e-3, lr_let=1e-2,
                 beta1=0.9, beta2=0.999, adam_eps=1e-8, weight_decay=0.0, timer=None,
                 group=0, nonfinite=None):
        super().__init__(ctypes.sizeof(BlockDesc), T, d, n_q, n_kv, head_dim, F, wbits, abits,
                         int(ffn_only), eps, rope_theta, optimizer, lr_lwc, lr_let, beta1,
                         beta2, adam_eps, weight_decay,
                         ctypes.pointer(timer.struct) if timer is not None else None, group,
                         nonfinite.data_ptr() if nonfinite is not None else None)


_SIGS = {
    "omq_status_str": (ctypes.c_char_p, [_int]),
    "omq_abi_version": (_int, []),
    "omq_lwc_fakequant": (_int, [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "omq_let_apply": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _int, _vp, _int, _i64, _vp,
                             _vp, _int, _vp, _vp]),
    "omq_act_quant": (_int, [_vp, _int, _i64, _i64, _int, _int, _vp, _vp, _vp, _int, _vp, _vp,
                             _vp, _vp, _vp, _vp, _vp]),
    "omq_gemm": (_int, [_i64, _i64, _i64, _vp, _i64, _int, _vp, _i64, _int, _int, _vp, _f, _vp,
                        _i64, _int, _vp]),
    "omq_code_gemm": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                             _vp, _vp, _vp, _i64, _vp]),
    "omq_code_gemm4": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                             _vp, _vp, _vp, _i64, _vp]),
    "omq_code_rowsum": (_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "omq_attention_fwd": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64,
                                 _vp, _vp]),
    "omq_attention_bwd_workspace_size": (_sz, [_i64, _i64, _i64]),
    "omq_attention_bwd": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp,
                                 _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _sz, _vp]),
    "omq_lwc_backward_workspace_size": (_sz, [_i64, _i64]),
    "omq_lwc_backward": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "omq_noalloc_scratch_bytes": (_sz, []),
    "omq_lwc_backward_noalloc": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "omq_act_quant_backward_workspace_size": (_sz, [_i64, _i64]),
    "omq_act_quant_backward": (_int, [_vp, _i64, _i64, _vp, _int, _int, _int, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "omq_qlinear_theta_size": (_i64, [ctypes.POINTER(QLinearDesc)]),
    "omq_qlinear_workspace_size": (_sz, [ctypes.POINTER(QLinearDesc)]),
    "omq_qlinear_fwd": (_int, [ctypes.POINTER(QLinearDesc), _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                               _vp]),
    "omq_qlinear_bwd": (_int, [ctypes.POINTER(QLinearDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _sz, _vp]),
    "omq_pack_codes": (_int, [_vp, _i64, _i64, _int, _vp, _vp]),
    "omq_fold_linear": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp]),
    "omq_w4a16_gemm": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp]),
    "omq_sgd": (_int, [_vp, _vp, _i64, _i64, _f, _f, _vp]),
    "omq_adamw": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _f, _f, _f, _f, _f, _f, _i64, _vp]),
    "omq_block_theta_layout": (_int, [ctypes.POINTER(BlockDesc), _vp, _vp, _vp, _vp]),
    "omq_block_workspace_size": (_sz, [ctypes.POINTER(BlockDesc)]),
    "omq_block_forward": (_int, [ctypes.POINTER(BlockDesc), _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "omq_block_step": (_int, [ctypes.POINTER(BlockDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _i64, _vp, _vp, _sz, _vp]),
}

_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libomq.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise OmqError("libomq.so not built: run `python -m post_quantization_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_str(rc: int) -> str:
    return lib().omq_status_str(rc).decode()


def abi_version() -> int:
    return lib().omq_abi_version()


def _check(name: str, rc: int) -> None:
    if rc != 0:
        raise OmqError("%s: %s (%d)" % (name, status_str(rc), rc))


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise OmqError("tensor must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise OmqError("unsupported dtype %s" % t.dtype)


def _tdt(code: int):
    return torch.float32 if code == F32 else torch.bfloat16


def _lwc_rows(c_out, c_in, group):
    return c_out * (c_in // group) if group and group != c_in else c_out


def lwc_fakequant(W, a_gamma, a_beta, n_bits, s=None, delta=None, B=None, out_dtype=None,
                  want_bias=False, want_codes=False, group=0,
                  nonfinite=None) -> Dict[str, torch.Tensor]:
    """nonfinite: optional int32 device tensor of one element, set to 1 when any
    element of the LET-transformed weight is NaN or infinite."""
    c_out, c_in = W.shape
    dev = W.device
    out_dtype = W.dtype if out_dtype is None else out_dtype
    rows = _lwc_rows(c_out, c_in, group)
    r = {"W_hat": torch.empty(c_out, c_in, dtype=out_dtype, device=dev),
         "h": torch.empty(rows, dtype=torch.float32, device=dev),
         "z": torch.empty(rows, dtype=torch.float32, device=dev),
         "arg_max": torch.empty(rows, dtype=torch.int32, device=dev),
         "arg_min": torch.empty(rows, dtype=torch.int32, device=dev)}
    r["B_tilde"] = torch.empty(c_out, dtype=torch.float32, device=dev) if want_bias else None
    r["codes"] = torch.empty(c_out, c_in, dtype=torch.uint8, device=dev) if want_codes else None
    _check("omq_lwc_fakequant", lib().omq_lwc_fakequant(
        _p(W), _dt(W), c_out, c_in, group, n_bits, _p(a_gamma), _p(a_beta), _p(s), _p(delta),
        _p(B),
        _p(r["W_hat"]), _dt(r["W_hat"]), _p(r["h"]), _p(r["z"]), _p(r["arg_max"]),
        _p(r["arg_min"]), _p(r["B_tilde"]), _p(r["codes"]), _p(nonfinite), _stream()))
    return r


def let_apply(s, delta=None, X=None, W=None, B=None, x_out_dtype=torch.float32,
              w_out_dtype=torch.float32, want_bias=False):
    dev = s.device
    c_in = s.numel()
    Xt = torch.empty(X.shape, dtype=x_out_dtype, device=dev) if X is not None else None
    Wt = torch.empty(W.shape, dtype=w_out_dtype, device=dev) if W is not None else None
    Bt = torch.empty(W.shape[0], dtype=torch.float32, device=dev) if (W is not None and want_bias) else None
    T = X.shape[0] if X is not None else 0
    c_out = W.shape[0] if W is not None else 0
    _check("omq_let_apply", lib().omq_let_apply(
        _p(X), _dt(X) if X is not None else 0, T, c_in, _p(s), _p(delta), _p(Xt),
        _dt(Xt) if Xt is not None else 0, _p(W), _dt(W) if W is not None else 0, c_out, _p(B),
        _p(Wt), _dt(Wt) if Wt is not None else 0, _p(Bt), _stream()))
    return Xt, Wt, Bt


def act_quant(X, n_bits, let_mode=LET_NONE, s=None, delta=None, out_dtype=torch.bfloat16,
              want_codes=False, nonfinite=None) -> Dict[str, torch.Tensor]:
    T, C = X.shape
    dev = X.device
    r = {"X_hat": torch.empty(T, C, dtype=out_dtype, device=dev),
         "h": torch.empty(T, dtype=torch.float32, device=dev),
         "z": torch.empty(T, dtype=torch.float32, device=dev),
         "arg_max": torch.empty(T, dtype=torch.int32, device=dev),
         "arg_min": torch.empty(T, dtype=torch.int32, device=dev)}
    r["codes"] = torch.empty(T, C, dtype=torch.uint8, device=dev) if want_codes else None
    _check("omq_act_quant", lib().omq_act_quant(
        _p(X), _dt(X), T, C, n_bits, let_mode, _p(s), _p(delta), _p(r["X_hat"]),
        _dt(r["X_hat"]), _p(r["h"]), _p(r["z"]), _p(r["arg_max"]), _p(r["arg_min"]),
        _p(r["codes"]), _p(nonfinite), _stream()))
    return r


def gemm(A, B, bias=None, alpha=1.0, C=None, accumulate=False, trans_a=False, trans_b=False):
    """C = alpha op(A) op(B)^T (+ bias) (+ C).  op(A) [M x K] is A, or A^T when trans_a
    (A stored [K x M]); op(B) [N x K] is B, or B^T when trans_b.  bf16 or float32."""
    K, M = A.shape if trans_a else A.shape[::-1]
    N = B.shape[1] if trans_b else B.shape[0]
    if C is None:
        C = torch.empty(M, N, dtype=torch.float32, device=A.device)
    _check("omq_gemm", lib().omq_gemm(M, N, K, _p(A), A.shape[1], int(trans_a), _p(B),
                                      B.shape[1], int(trans_b), _dt(A), _p(bias), alpha, _p(C),
                                      N, int(accumulate), _stream()))
    return C


def code_rowsum(codes):
    """int32 sums of each row of a uint8 code matrix."""
    rows, cols = codes.shape
    sums = torch.empty(rows, dtype=torch.int32, device=codes.device)
    _check("omq_code_rowsum", lib().omq_code_rowsum(_p(codes), rows, cols, cols, _p(sums),
                                                    _stream()))
    return sums


def code_gemm(qa, h_a, z_a, qb, h_b, z_b, sum_a=None, sum_b=None, bias=None, C=None):
    """C = ((qa - z_a) h_a) ((qb - z_b) h_b)^T + bias from uint8 codes qa [M x K], qb
    [N x K] with per-row steps and zero points; the code sums default to
    code_rowsum of each operand."""
    M, K = qa.shape
    N = qb.shape[0]
    if sum_a is None:
        sum_a = code_rowsum(qa)
    if sum_b is None:
        sum_b = code_rowsum(qb)
    if C is None:
        C = torch.empty(M, N, dtype=torch.float32, device=qa.device)
    _check("omq_code_gemm", lib().omq_code_gemm(
        M, N, K, _p(qa), K, _p(h_a), _p(z_a), _p(sum_a), _p(qb), K, _p(h_b), _p(z_b), _p(sum_b),
        _p(bias), _p(C), N, _stream()))
    return C


def code_gemm4(qa, h_a, z_a, qb, h_b, z_b, K, sum_a, sum_b, bias=None, C=None):
    """code_gemm on 4-bit codes packed two to a byte (uint8 [M x K/2], [N x K/2], the
    low nibble first); K is the number of codes per row, sum_a / sum_b their sums."""
    M, N = qa.shape[0], qb.shape[0]
    if C is None:
        C = torch.empty(M, N, dtype=torch.float32, device=qa.device)
    _check("omq_code_gemm4", lib().omq_code_gemm4(
        M, N, K, _p(qa), qa.shape[1], _p(h_a), _p(z_a), _p(sum_a), _p(qb), qb.shape[1], _p(h_b),
        _p(z_b), _p(sum_b), _p(bias), _p(C), N, _stream()))
    return C


def attention_fwd(Q, K, V, n_q, n_kv, head_dim=128):
    """Causal attention of bf16 Q [T x n_q*hd], K, V [T x n_kv*hd]: returns O (float32
    [T x n_q*hd]) and the base-2 log-sum-exp per (head, query) [n_q x T]."""
    T = Q.shape[0]
    O = torch.empty(T, n_q * head_dim, dtype=torch.float32, device=Q.device)
    lse2 = torch.empty(n_q, T, dtype=torch.float32, device=Q.device)
    _check("omq_attention_fwd", lib().omq_attention_fwd(
        _p(Q), Q.shape[1], _p(K), _p(V), K.shape[1], T, n_q, n_kv, head_dim, _p(O), O.shape[1],
        _p(lse2), _stream()))
    return O, lse2


def attention_bwd(Q, K, V, O, lse2, dO, n_q, n_kv, head_dim=128):
    """Backward of attention_fwd given dO (float32 like O): (dQ, dK, dV) float32."""
    T = Q.shape[0]
    dQ = torch.empty(T, n_q * head_dim, dtype=torch.float32, device=Q.device)
    dK = torch.empty(T, n_kv * head_dim, dtype=torch.float32, device=Q.device)
    dV = torch.empty_like(dK)
    nbytes = lib().omq_attention_bwd_workspace_size(T, n_q, Q.shape[1])
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=Q.device)
    _check("omq_attention_bwd", lib().omq_attention_bwd(
        _p(Q), Q.shape[1], _p(K), _p(V), K.shape[1], T, n_q, n_kv, head_dim, _p(O), _p(dO),
        O.shape[1], _p(lse2), _p(dQ), dQ.shape[1], _p(dK), _p(dV), dK.shape[1], _p(ws), nbytes,
        _stream()))
    return dQ, dK, dV


def lwc_backward(gW_hat, W, n_bits, a_gamma, a_beta, h, z, arg_max, arg_min, s=None,
                 dy_colsum=None, want_s=False, want_delta=False, group=0):
    c_out, c_in = W.shape
    dev = W.device
    rows = _lwc_rows(c_out, c_in, group)
    ga = torch.empty(rows, dtype=torch.float32, device=dev)
    gb = torch.empty(rows, dtype=torch.float32, device=dev)
    gs = torch.empty(c_in, dtype=torch.float32, device=dev) if want_s else None
    gd = torch.empty(c_in, dtype=torch.float32, device=dev) if want_delta else None
    nbytes = lib().omq_lwc_backward_workspace_size(c_out, c_in)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check("omq_lwc_backward", lib().omq_lwc_backward(
        _p(gW_hat), _p(W), _dt(W), c_out, c_in, group, n_bits, _p(a_gamma), _p(a_beta), _p(s),
        _p(h),
        _p(z), _p(arg_max), _p(arg_min), _p(dy_colsum), _p(ga), _p(gb), _p(gs), _p(gd), _p(ws),
        nbytes, _stream()))
    return ga, gb, gs, gd


def noalloc_scratch_bytes() -> int:
    return lib().omq_noalloc_scratch_bytes()


def lwc_backward_noalloc(gW_hat, W, n_bits, a_gamma, a_beta, h, z, arg_max, arg_min, s=None,
                         dy_colsum=None, want_s=False, want_delta=False, group=0, out=None):
    """lwc_backward with the library's fixed device scratch (no workspace allocation
    inside the library).  out: optional (ga, gb, gs, gd) tensors to write into."""
    c_out, c_in = W.shape
    dev = W.device
    rows = _lwc_rows(c_out, c_in, group)
    if out is None:
        ga = torch.empty(rows, dtype=torch.float32, device=dev)
        gb = torch.empty(rows, dtype=torch.float32, device=dev)
        gs = torch.empty(c_in, dtype=torch.float32, device=dev) if want_s else None
        gd = torch.empty(c_in, dtype=torch.float32, device=dev) if want_delta else None
    else:
        ga, gb, gs, gd = out
    _check("omq_lwc_backward_noalloc", lib().omq_lwc_backward_noalloc(
        _p(gW_hat), _p(W), _dt(W), c_out, c_in, group, n_bits, _p(a_gamma), _p(a_beta), _p(s),
        _p(h), _p(z), _p(arg_max), _p(arg_min), _p(dy_colsum), _p(ga), _p(gb), _p(gs), _p(gd),
        _stream()))
    return ga, gb, gs, gd


def act_quant_backward(gX_hat, X, n_bits, h, z, arg_max, arg_min, let_mode=LET_NONE, s=None,
                       delta=None, want_gx=True, want_s=False, want_delta=False):
    T, C = X.shape
    dev = X.device
    gx = torch.empty(T, C, dtype=torch.float32, device=dev) if want_gx else None
    gs = torch.empty(C, dtype=torch.float32, device=dev) if want_s else None
    gd = torch.empty(C, dtype=torch.float32, device=dev) if want_delta else None
    nbytes = lib().omq_act_quant_backward_workspace_size(T, C)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check("omq_act_quant_backward", lib().omq_act_quant_backward(
        _p(gX_hat), T, C, _p(X), _dt(X), n_bits, let_mode, _p(s), _p(delta), _p(h), _p(z),
        _p(arg_max), _p(arg_min), _p(gx), _p(gs), _p(gd), _p(ws), nbytes, _stream()))
    return gx, gs, gd


def qlinear_theta_size(desc: QLinearDesc) -> int:
    return lib().omq_qlinear_theta_size(ctypes.byref(desc))


def qlinear_workspace_size(desc: QLinearDesc) -> int:
    return lib().omq_qlinear_workspace_size(ctypes.byref(desc))


def qlinear_fwd(desc, X, W, B, theta, Y, ws):
    _check("omq_qlinear_fwd", lib().omq_qlinear_fwd(
        ctypes.byref(desc), _p(X), _p(W), _p(B), _p(theta), _p(Y), _p(ws), ws.numel(), _stream()))
    return Y


def qlinear_bwd(desc, X, W, theta, dY, dX, dtheta, ws):
    _check("omq_qlinear_bwd", lib().omq_qlinear_bwd(
        ctypes.byref(desc), _p(X), _p(W), _p(theta), _p(dY), _p(dX), _p(dtheta), _p(ws),
        ws.numel(), _stream()))
    return dtheta


def sgd(theta, grad, n_lwc, lr_lwc, lr_let):
    _check("omq_sgd", lib().omq_sgd(_p(theta), _p(grad), theta.numel(), n_lwc, lr_lwc, lr_let,
                                    _stream()))


def adamw(theta, grad, m, v, n_lwc, lr_lwc, lr_let, step, beta1=0.9, beta2=0.999, eps=1e-8,
          weight_decay=0.0):
    _check("omq_adamw", lib().omq_adamw(_p(theta), _p(grad), _p(m), _p(v), theta.numel(), n_lwc,
                                        lr_lwc, lr_let, beta1, beta2, eps, weight_decay, step,
                                        _stream()))


def block_theta_layout(desc: BlockDesc):
    """(offsets of the packed entries, number of leading LWC logits, total size)."""
    offs = (ctypes.c_int64 * 32)()
    n = ctypes.c_int64()
    nl = ctypes.c_int64()
    tot = ctypes.c_int64()
    _check("omq_block_theta_layout", lib().omq_block_theta_layout(
        ctypes.byref(desc), ctypes.addressof(offs), ctypes.addressof(n), ctypes.addressof(nl),
        ctypes.addressof(tot)))
    return list(offs[:n.value]), nl.value, tot.value


def block_workspace_size(desc: BlockDesc) -> int:
    return lib().omq_block_workspace_size(ctypes.byref(desc))


def _wptrs(weights: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * 7)()
    for i, w in enumerate(weights):
        arr[i] = _p(w) if w is not None else None
    return arr


def block_forward(desc, x, weights, theta, y, ws):
    arr = _wptrs(weights)
    _check("omq_block_forward", lib().omq_block_forward(
        ctypes.byref(desc), _p(x), ctypes.addressof(arr), _p(theta), _p(y), _p(ws), ws.numel(),
        _stream()))
    return y


def block_step(desc, x, y_target, weights, theta, dtheta, adam_m, adam_v, step, loss, ws):
    arr = _wptrs(weights)
    _check("omq_block_step", lib().omq_block_step(
        ctypes.byref(desc), _p(x), _p(y_target), ctypes.addressof(arr), _p(theta), _p(dtheta),
        _p(adam_m), _p(adam_v), step, _p(loss), _p(ws), ws.numel(), _stream()))


# ---------------------------------------------------------------------------
# deployment form
# ---------------------------------------------------------------------------

def pack_codes(codes: torch.Tensor, n_bits: int) -> torch.Tensor:
    """uint8 codes [rows x cols] -> packed int32 words [rows x ceil(cols / (32 // n_bits))]."""
    rows, cols = codes.shape
    per = 32 // n_bits
    words = torch.empty(rows, (cols + per - 1) // per, dtype=torch.int32, device=codes.device)
    _check("omq_pack_codes", lib().omq_pack_codes(_p(codes), rows, cols, n_bits, _p(words),
                                                   _stream()))
    return words


def fold_linear(words, n_bits, N, K, h, z, group=0, B=None, s=None, delta=None, s_o=None,
                delta_o=None, want_gain=False):
    """Weight-only LET fold: returns (bias_out [N], h_out or None), and the input
    site's gain 1/s [K] as a third item when want_gain."""
    dev = words.device
    bias = torch.empty(N, dtype=torch.float32, device=dev)
    h_out = torch.empty_like(h) if s_o is not None else None
    gain = torch.empty(K, dtype=torch.float32, device=dev) if want_gain else None
    _check("omq_fold_linear", lib().omq_fold_linear(
        _p(words), n_bits, N, K, _p(h), _p(z), group, _p(B), _p(s), _p(delta), _p(s_o),
        _p(delta_o), _p(bias), _p(h_out), _p(gain), _stream()))
    return (bias, h_out, gain) if want_gain else (bias, h_out)


def w4a16_gemm(X, words, N, h, z, group=0, bias=None, Y=None):
    """Y [T x N] float32 = X (bf16 [T x K]) W_hat^T + bias from packed 4-bit codes."""
    T, K = X.shape
    if Y is None:
        Y = torch.empty(T, N, dtype=torch.float32, device=X.device)
    _check("omq_w4a16_gemm", lib().omq_w4a16_gemm(
        _p(X), T, K, _p(words), N, _p(h), _p(z), group, _p(bias), _p(Y), _stream()))
    return Y
