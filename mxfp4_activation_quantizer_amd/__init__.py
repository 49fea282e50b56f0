"""Python binding of libkq.so, the KroQuant MXFP4 activation quantizer for MI355X.

Argument marshalling only: every computation runs in the HIP kernels of
libkq.so (include/kq.h documents the C ABI). PyTorch provides device memory
and streams. There is no CPU fallback: if the library is missing or the
device is not a GPU, the calls raise.

Method: KroQuant (arXiv 2607.21446v1), Sec. 3.1-3.2 and 3.5 (Eq. 1, 4, 5, 12),
with the MXFP4 format of Sec. 4.1 / Appendix D.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkq.so")

KQ_OK, KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_HIP, KQ_ERR_UNSUPPORTED = range(6)

# Every symbol include/kq.h declares.
EXPORTS = (
    "kq_quantize_mxfp4",
    "kq_transform_quantize_mxfp4",
    "kq_transform_quantize_mxfp4_form",
    "kq_smoothquant_quantize_mxfp4",
    "kq_quantize_mxfp4_f32",
    "kq_inverse_fold_weights",
    "kq_mxfp4_gemm",
    "kq_mxfp4_gemm_wide",
    "kq_pack_mxfp4_scales",
    "kq_lowrank_project_bf16",
    "kq_lowrank_project_bf16_split",
    "kq_lowrank_project_split",
    "kq_dequantize_mxfp4_bf16",
    "kq_mxfp4_gemm_packed",
    "kq_mxfp4_gemm_packed_bf16",
    "kq_mxfp4_gemm_packed_lowrank",
    "kq_mxfp4_gemm_packed_lowrank_split",
    "kq_transform_quantize_mxfp4_gemm",
    "kq_hadamard_quantize_mxfp4",
    "kq_transform_quantize_mxfp4_y16",
    "kq_transform_quantize_mxfp4_packed",
    "kq_lowrank_project",
    "kq_mxfp4_gemm_lowrank",
    "kq_gemm_f32",
    "kq_calib_workspace_bytes",
    "kq_calib_init",
    "kq_calib_step",
    "kq_calib_step_noalloc",
    "kq_status_string",
    "kq_last_hip_error",
    "kq_factors_from_lu",
)

_lib = None


class KQError(RuntimeError):
    def __init__(self, fn, status, lib):
        msg = lib.kq_status_string(status).decode()
        if status == KQ_ERR_HIP:
            msg += " (hipError_t %d)" % lib.kq_last_hip_error()
        super().__init__("%s: %s" % (fn, msg))
        self.status = status


def lib():
    """Load libkq.so (built by ``__graft_entry__.build()`` or ``python -m ...build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkq.so is not built: run `python -m mxfp4_activation_quantizer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for name, args in {
            "kq_quantize_mxfp4": [p, i64, i64, i64, p, p, p],
            "kq_transform_quantize_mxfp4": [p, i64, i64, i64, p, p, p, p, p],
            "kq_transform_quantize_mxfp4_form": [p, i64, i64, i64, p, p, p, p, st, p],
            "kq_smoothquant_quantize_mxfp4": [p, i64, i64, i64, p, p, p, p],
            "kq_quantize_mxfp4_f32": [p, i64, i64, i64, p, p, p],
            "kq_inverse_fold_weights": [p, i64, i64, p, p, p],
            "kq_factors_from_lu": [p, i64, p],
            "kq_mxfp4_gemm": [p, p, p, p, i64, i64, i64, p, i64, p],
            "kq_mxfp4_gemm_wide": [p, p, p, p, i64, i64, i64, p, i64, p],
            "kq_pack_mxfp4_scales": [p, i64, i64, p, p],
            "kq_lowrank_project_bf16": [p, i64, i64, i64, p, i64, p, p],
            "kq_lowrank_project_bf16_split": [p, i64, i64, i64, p, i64, p, p, p],
            "kq_lowrank_project_split": [p, i64, i64, i64, p, p, i64, p, p, p],
            "kq_dequantize_mxfp4_bf16": [p, p, i64, i64, p, p],
            "kq_mxfp4_gemm_packed": [p, p, p, p, i64, i64, i64, p, i64, p],
            "kq_mxfp4_gemm_packed_bf16": [p, p, p, p, i64, i64, i64, p, i64, p],
            "kq_mxfp4_gemm_packed_lowrank": [p, p, p, p, i64, i64, i64, p, p, p, i64, p, i64, p],
            "kq_mxfp4_gemm_packed_lowrank_split": [p, p, p, p, i64, i64, i64, p, p, p, i64, p, i64, p],
            "kq_transform_quantize_mxfp4_gemm": [p, i64, i64, i64, p, p, p, i64, p, i64, p],
            "kq_hadamard_quantize_mxfp4": [p, i64, i64, i64, i64, p, p, p, p],
            "kq_transform_quantize_mxfp4_y16": [p, i64, i64, i64, p, p, p, p, p],
            "kq_transform_quantize_mxfp4_packed": [p, i64, i64, i64, p, p, p, p, p],
            "kq_lowrank_project": [p, i64, i64, i64, p, p, i64, p, p],
            "kq_mxfp4_gemm_lowrank": [p, p, p, p, i64, i64, i64, p, p, p, i64, p, i64, p],
            "kq_gemm_f32": [st, st, i64, i64, i64, ctypes.c_float, p, i64, p, i64, ctypes.c_float, p, i64, p,
                            i64, p],
            "kq_calib_workspace_bytes": [i64, i64, i64, p],
            "kq_calib_init": [p, i64, i64, p, i64, p, i64, p],
            "kq_calib_step": [p, i64, i64, i64, p, p, p, i64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                              ctypes.c_float, p, st, p, p, p, i64, p],
            "kq_calib_step_noalloc": [p, p, i64, i64, i64, p, p, p, i64, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_float, ctypes.c_float, p, st, p, p, p],
        }.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = st
        L.kq_status_string.argtypes = [st]
        L.kq_status_string.restype = ctypes.c_char_p
        L.kq_last_hip_error.argtypes = []
        L.kq_last_hip_error.restype = st
        _lib = L
    return _lib


def _check(fn, status):
    if status != KQ_OK:
        raise KQError(fn, status, lib())


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtypes):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    return t


def _rows(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("%s must be 2-D with unit column stride" % name)
    return t.shape[0], t.shape[1], t.stride(0)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _outputs(m, d, device, codes, scales):
    torch = _torch()
    if codes is None:
        codes = torch.empty((m, d // 2), dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty((m, d // 32), dtype=torch.uint8, device=device)
    _dev(codes, "codes", (torch.uint8,))
    _dev(scales, "scales", (torch.uint8,))
    if tuple(codes.shape) != (m, d // 2) or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous [m][d/2] uint8 tensor")
    if tuple(scales.shape) != (m, d // 32) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous [m][d/32] uint8 tensor")
    return codes, scales


def _bf16_input(A):
    torch = _torch()
    _dev(A, "A", (torch.bfloat16, torch.int16, torch.uint16))
    return _rows(A, "A")


def quantize_mxfp4(A, codes=None, scales=None, stream=None):
    """MXFP4 codes [m][d/2] and E8M0 scales [m][d/32] of bf16 A [m][d] (T = I)."""
    m, d, lda = _bf16_input(A)
    codes, scales = _outputs(m, d, A.device, codes, scales)
    _check("kq_quantize_mxfp4",
           lib().kq_quantize_mxfp4(_p(A), m, d, lda, _p(codes), _p(scales), _stream_ptr(stream)))
    return codes, scales


FORMS = {"butterfly": 0, "mfma": 1, "mfma_lds": 2}  # kq_transform_form


def transform_quantize_mxfp4(A, factors, codes=None, scales=None, y_debug=None, stream=None, form=None):
    """Fused y = A T (per-block Kronecker factors fp32 [d/32][5][2][2]) then MXFP4.

    ``y_debug``: optional fp32 [m][d] tensor that receives y (check mode).
    ``form``: None (the library's default, the butterfly form) or one of FORMS.
    """
    torch = _torch()
    m, d, lda = _bf16_input(A)
    _dev(factors, "factors", (torch.float32,))
    if factors.numel() != (d // 32) * 20 or not factors.is_contiguous():
        raise ValueError("factors must be contiguous fp32 [d/32][5][2][2]")
    if y_debug is not None:
        _dev(y_debug, "y_debug", (torch.float32,))
        if tuple(y_debug.shape) != (m, d) or not y_debug.is_contiguous():
            raise ValueError("y_debug must be a contiguous fp32 [m][d] tensor")
    codes, scales = _outputs(m, d, A.device, codes, scales)
    if form is None:
        _check("kq_transform_quantize_mxfp4",
               lib().kq_transform_quantize_mxfp4(_p(A), m, d, lda, _p(factors), _p(codes), _p(scales),
                                                 _p(y_debug), _stream_ptr(stream)))
    else:
        _check("kq_transform_quantize_mxfp4_form",
               lib().kq_transform_quantize_mxfp4_form(_p(A), m, d, lda, _p(factors), _p(codes), _p(scales),
                                                      _p(y_debug), FORMS[form], _stream_ptr(stream)))
    return codes, scales


def hadamard_quantize_mxfp4(A, n, codes=None, scales=None, y_debug=None, stream=None):
    """Block-Hadamard baseline: each group of n channels times H_n / sqrt(n), then MXFP4.

    n = 32 is the block-size Hadamard, n = d the full-width transform (FWHT).
    """
    torch = _torch()
    m, d, lda = _bf16_input(A)
    if y_debug is not None:
        _dev(y_debug, "y_debug", (torch.float32,))
        if tuple(y_debug.shape) != (m, d) or not y_debug.is_contiguous():
            raise ValueError("y_debug must be a contiguous fp32 [m][d] tensor")
    codes, scales = _outputs(m, d, A.device, codes, scales)
    _check("kq_hadamard_quantize_mxfp4",
           lib().kq_hadamard_quantize_mxfp4(_p(A), m, d, lda, int(n), _p(codes), _p(scales),
                                            _p(y_debug), _stream_ptr(stream)))
    return codes, scales


def transform_quantize_mxfp4_y16(A, factors, codes=None, scales=None, y16=None, stream=None):
    """Fused y = A T then MXFP4, also writing bf16(y) [m][d] (the 16-bit activation the
    low-rank branch of Eq. 11 consumes). Returns codes, scales, y16."""
    torch = _torch()
    m, d, lda = _bf16_input(A)
    _dev(factors, "factors", (torch.float32,))
    if factors.numel() != (d // 32) * 20 or not factors.is_contiguous():
        raise ValueError("factors must be contiguous fp32 [d/32][5][2][2]")
    if y16 is None:
        y16 = torch.empty((m, d), dtype=torch.bfloat16, device=A.device)
    _dev(y16, "y16", (torch.bfloat16,))
    if tuple(y16.shape) != (m, d) or not y16.is_contiguous():
        raise ValueError("y16 must be a contiguous bf16 [m][d] tensor")
    codes, scales = _outputs(m, d, A.device, codes, scales)
    _check("kq_transform_quantize_mxfp4_y16",
           lib().kq_transform_quantize_mxfp4_y16(_p(A), m, d, lda, _p(factors), _p(codes), _p(scales), _p(y16),
                                                 _stream_ptr(stream)))
    return codes, scales, y16


def transform_quantize_mxfp4_packed(A, factors, codes=None, packed_scales=None, y16=None, want_y16=False,
                                     stream=None):
    """Fused y = A T then MXFP4 with the scales written in the packed-GEMM layout
    [d/256][m][8] (what pack_mxfp4_scales makes of them; d % 256 == 0), optionally also
    bf16(y) [m][d] (y16, or want_y16=True to allocate it). Returns codes, packed scales, y16
    (or None)."""
    torch = _torch()
    m, d, lda = _bf16_input(A)
    _dev(factors, "factors", (torch.float32,))
    if factors.numel() != (d // 32) * 20 or not factors.is_contiguous():
        raise ValueError("factors must be contiguous fp32 [d/32][5][2][2]")
    if codes is None:
        codes = torch.empty((m, d // 2), dtype=torch.uint8, device=A.device)
    _dev(codes, "codes", (torch.uint8,))
    if tuple(codes.shape) != (m, d // 2) or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous [m][d/2] uint8 tensor")
    if packed_scales is None:
        packed_scales = torch.empty((d // 256 if d % 256 == 0 else 0, m, 8), dtype=torch.uint8, device=A.device)
    _dev(packed_scales, "packed_scales", (torch.uint8,))
    if packed_scales.numel() != m * (d // 32) or not packed_scales.is_contiguous():
        raise ValueError("packed_scales must be a contiguous uint8 tensor of m * d/32 bytes")
    if y16 is None and want_y16:
        y16 = torch.empty((m, d), dtype=torch.bfloat16, device=A.device)
    if y16 is not None:
        _dev(y16, "y16", (torch.bfloat16,))
        if tuple(y16.shape) != (m, d) or not y16.is_contiguous():
            raise ValueError("y16 must be a contiguous bf16 [m][d] tensor")
    _check("kq_transform_quantize_mxfp4_packed",
           lib().kq_transform_quantize_mxfp4_packed(_p(A), m, d, lda, _p(factors), _p(codes), _p(packed_scales),
                                                    _p(y16) if y16 is not None else None, _stream_ptr(stream)))
    return codes, packed_scales, y16


def lowrank_project(X16, codes_r, scales_r, out=None, stream=None):
    """Z = X16 Q(R)^T in fp32: X16 bf16 [m][d], R in MXFP4 (codes [r][d/2], scales [r][d/32])."""
    torch = _torch()
    _dev(X16, "X16", (torch.bfloat16, torch.int16, torch.uint16))
    m, d, ldx = _rows(X16, "X16")
    for t, nm in ((codes_r, "codes_r"), (scales_r, "scales_r")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    r = codes_r.shape[0]
    if tuple(codes_r.shape) != (r, d // 2) or tuple(scales_r.shape) != (r, d // 32):
        raise ValueError("R operand shapes do not match X16")
    if out is None:
        out = torch.empty((m, r), dtype=torch.float32, device=X16.device)
    _dev(out, "out", (torch.float32,))
    if tuple(out.shape) != (m, r) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [m][r] tensor")
    _check("kq_lowrank_project",
           lib().kq_lowrank_project(_p(X16), m, d, ldx, _p(codes_r), _p(scales_r), r, _p(out), _stream_ptr(stream)))
    return out


def lowrank_project_split(X16, codes_r, scales_r, Zh=None, Zl=None, stream=None):
    """As lowrank_project (R in MXFP4), Z written as its bf16 split: Zh = bf16(Z),
    Zl = bf16(Z - Zh) (bf16 [m][r] each). Returns Zh, Zl."""
    torch = _torch()
    _dev(X16, "X16", (torch.bfloat16, torch.int16, torch.uint16))
    m, d, ldx = _rows(X16, "X16")
    for t, nm in ((codes_r, "codes_r"), (scales_r, "scales_r")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    r = codes_r.shape[0]
    if tuple(codes_r.shape) != (r, d // 2) or tuple(scales_r.shape) != (r, d // 32):
        raise ValueError("R operand shapes do not match X16")
    outs = []
    for t, nm in ((Zh, "Zh"), (Zl, "Zl")):
        if t is None:
            t = torch.empty((m, r), dtype=torch.bfloat16, device=X16.device)
        _dev(t, nm, (torch.bfloat16,))
        if tuple(t.shape) != (m, r) or not t.is_contiguous():
            raise ValueError(nm + " must be a contiguous bf16 [m][r] tensor")
        outs.append(t)
    Zh, Zl = outs
    _check("kq_lowrank_project_split",
           lib().kq_lowrank_project_split(_p(X16), m, d, ldx, _p(codes_r), _p(scales_r), r, _p(Zh), _p(Zl),
                                          _stream_ptr(stream)))
    return Zh, Zl


def dequantize_mxfp4_bf16(codes, scales, out=None, stream=None):
    """deq(codes, scales) as bf16 [rows][k] (exact): codes [rows][k/2], scales [rows][k/32]."""
    torch = _torch()
    for t, nm in ((codes, "codes"), (scales, "scales")):
        _dev(t, nm, (torch.uint8,))
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(nm + " must be a contiguous 2-D uint8 tensor")
    rows, kb = codes.shape
    k = kb * 2
    if tuple(scales.shape) != (rows, k // 32):
        raise ValueError("scales must be [rows][k/32]")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.bfloat16, device=codes.device)
    _dev(out, "out", (torch.bfloat16, torch.int16, torch.uint16))
    if tuple(out.shape) != (rows, k) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [rows][k] tensor")
    _check("kq_dequantize_mxfp4_bf16",
           lib().kq_dequantize_mxfp4_bf16(_p(codes), _p(scales), rows, k, _p(out), _stream_ptr(stream)))
    return out


def lowrank_project_bf16(X16, R16, out=None, stream=None):
    """Z = X16 R16^T in fp32: X16 bf16 [m][d], R16 bf16 [r][d] (e.g. dequantize_mxfp4_bf16 of R)."""
    torch = _torch()
    _dev(X16, "X16", (torch.bfloat16, torch.int16, torch.uint16))
    _dev(R16, "R16", (torch.bfloat16, torch.int16, torch.uint16))
    m, d, ldx = _rows(X16, "X16")
    if R16.dim() != 2 or R16.shape[1] != d or not R16.is_contiguous():
        raise ValueError("R16 must be a contiguous bf16 [r][d] tensor")
    r = R16.shape[0]
    if out is None:
        out = torch.empty((m, r), dtype=torch.float32, device=X16.device)
    _dev(out, "out", (torch.float32,))
    if tuple(out.shape) != (m, r) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [m][r] tensor")
    _check("kq_lowrank_project_bf16",
           lib().kq_lowrank_project_bf16(_p(X16), m, d, ldx, _p(R16), r, _p(out), _stream_ptr(stream)))
    return out


def lowrank_project_bf16_split(X16, R16, Zh=None, Zl=None, stream=None):
    """As lowrank_project_bf16, Z written as its bf16 split: Zh = bf16(Z), Zl = bf16(Z - Zh)
    (bf16 [m][r] each). Returns Zh, Zl."""
    torch = _torch()
    _dev(X16, "X16", (torch.bfloat16, torch.int16, torch.uint16))
    _dev(R16, "R16", (torch.bfloat16, torch.int16, torch.uint16))
    m, d, ldx = _rows(X16, "X16")
    if R16.dim() != 2 or R16.shape[1] != d or not R16.is_contiguous():
        raise ValueError("R16 must be a contiguous bf16 [r][d] tensor")
    r = R16.shape[0]
    outs = []
    for t, nm in ((Zh, "Zh"), (Zl, "Zl")):
        if t is None:
            t = torch.empty((m, r), dtype=torch.bfloat16, device=X16.device)
        _dev(t, nm, (torch.bfloat16,))
        if tuple(t.shape) != (m, r) or not t.is_contiguous():
            raise ValueError(nm + " must be a contiguous bf16 [m][r] tensor")
        outs.append(t)
    Zh, Zl = outs
    _check("kq_lowrank_project_bf16_split",
           lib().kq_lowrank_project_bf16_split(_p(X16), m, d, ldx, _p(R16), r, _p(Zh), _p(Zl), _stream_ptr(stream)))
    return Zh, Zl


def mxfp4_gemm_lowrank(codes_a, scales_a, codes_w, scales_w, Z, codes_l, scales_l, out=None, stream=None):
    """O = deq(A) deq(W)^T + Z deq(L)^T (Eq. 11's two terms): Z fp32 [m][r], L in MXFP4
    (codes [n][r/2], scales [n][r/32])."""
    torch = _torch()
    for t, nm in ((codes_a, "codes_a"), (scales_a, "scales_a"), (codes_w, "codes_w"), (scales_w, "scales_w"),
                  (codes_l, "codes_l"), (scales_l, "scales_l")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    _dev(Z, "Z", (torch.float32,))
    m, kb = codes_a.shape
    n = codes_w.shape[0]
    k = kb * 2
    r = Z.shape[1]
    if tuple(codes_w.shape) != (n, kb) or tuple(scales_a.shape) != (m, k // 32) or \
            tuple(scales_w.shape) != (n, k // 32) or Z.shape[0] != m or not Z.is_contiguous() or \
            tuple(codes_l.shape) != (n, r // 2) or tuple(scales_l.shape) != (n, r // 32):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=codes_a.device)
    _dev(out, "out", (torch.float32,))
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError("out must be fp32 [m][n] with unit column stride")
    _check("kq_mxfp4_gemm_lowrank",
           lib().kq_mxfp4_gemm_lowrank(_p(codes_a), _p(scales_a), _p(codes_w), _p(scales_w), m, n, k, _p(Z),
                                       _p(codes_l), _p(scales_l), r, _p(out), out.stride(0), _stream_ptr(stream)))
    return out


def smoothquant_quantize_mxfp4(A, inv_scale, codes=None, scales=None, stream=None):
    """SmoothQuant baseline: y_c = fl32(a_c * inv_scale[c]) then MXFP4."""
    torch = _torch()
    m, d, lda = _bf16_input(A)
    _dev(inv_scale, "inv_scale", (torch.float32,))
    if inv_scale.numel() < d or not inv_scale.is_contiguous():
        raise ValueError("inv_scale must be a contiguous fp32 vector of length d")
    codes, scales = _outputs(m, d, A.device, codes, scales)
    _check("kq_smoothquant_quantize_mxfp4",
           lib().kq_smoothquant_quantize_mxfp4(_p(A), m, d, lda, _p(inv_scale), _p(codes),
                                               _p(scales), _stream_ptr(stream)))
    return codes, scales


def quantize_mxfp4_f32(X, codes=None, scales=None, stream=None):
    """MXFP4 codes and scales of fp32 X [m][d]."""
    torch = _torch()
    _dev(X, "X", (torch.float32,))
    m, d, ldx = _rows(X, "X")
    codes, scales = _outputs(m, d, X.device, codes, scales)
    _check("kq_quantize_mxfp4_f32",
           lib().kq_quantize_mxfp4_f32(_p(X), m, d, ldx, _p(codes), _p(scales), _stream_ptr(stream)))
    return codes, scales


def inverse_fold_weights(W, factors, out=None, stream=None):
    """W' = W T^{-T} for fp32 W [o][d] (the weight side of Eq. 1)."""
    torch = _torch()
    _dev(W, "W", (torch.float32,))
    _dev(factors, "factors", (torch.float32,))
    if not W.is_contiguous():
        raise ValueError("W must be contiguous")
    o, d = W.shape
    if factors.numel() != (d // 32) * 20 or not factors.is_contiguous():
        raise ValueError("factors must be contiguous fp32 [d/32][5][2][2]")
    if out is None:
        out = torch.empty_like(W)
    _dev(out, "out", (torch.float32,))
    if out.shape != W.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like W")
    _check("kq_inverse_fold_weights",
           lib().kq_inverse_fold_weights(_p(W), o, d, _p(factors), _p(out), _stream_ptr(stream)))
    return out


def _gemm_operands(codes_a, scales_a, codes_w, scales_w, out):
    torch = _torch()
    for t, nm in ((codes_a, "codes_a"), (scales_a, "scales_a"), (codes_w, "codes_w"), (scales_w, "scales_w")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    m, kb = codes_a.shape
    n = codes_w.shape[0]
    k = kb * 2
    if tuple(codes_w.shape) != (n, kb) or tuple(scales_a.shape) != (m, k // 32) or \
            tuple(scales_w.shape) != (n, k // 32):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=codes_a.device)
    _dev(out, "out", (torch.float32,))
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError("out must be fp32 [m][n] with unit column stride")
    return m, n, k, out


def mxfp4_gemm(codes_a, scales_a, codes_w, scales_w, out=None, stream=None):
    """O = deq(A) deq(W)^T in fp32 from MXFP4 operands (codes [rows][k/2], scales [rows][k/32])."""
    m, n, k, out = _gemm_operands(codes_a, scales_a, codes_w, scales_w, out)
    _check("kq_mxfp4_gemm",
           lib().kq_mxfp4_gemm(_p(codes_a), _p(scales_a), _p(codes_w), _p(scales_w), m, n, k, _p(out),
                               out.stride(0), _stream_ptr(stream)))
    return out


def pack_mxfp4_scales(scales, out=None, stream=None):
    """MXFP4 scales [rows][k/32] -> the GEMM-ready layout [k/256][rows][8] (k % 256 == 0)."""
    torch = _torch()
    _dev(scales, "scales", (torch.uint8,))
    if scales.dim() != 2 or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous [rows][k/32] uint8 tensor")
    rows, kb = scales.shape
    k = kb * 32
    if out is None:
        out = torch.empty((kb // 8 if kb % 8 == 0 else 0, rows, 8), dtype=torch.uint8, device=scales.device)
    _dev(out, "out", (torch.uint8,))
    if out.numel() != rows * kb or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 tensor of rows * k/32 bytes")
    _check("kq_pack_mxfp4_scales",
           lib().kq_pack_mxfp4_scales(_p(scales), rows, k, _p(out), _stream_ptr(stream)))
    return out


def mxfp4_gemm_packed(codes_a, packed_scales_a, codes_w, packed_scales_w, out=None, stream=None, bf16=False):
    """O = deq(A) deq(W)^T in fp32 (bf16=True: rounded to bf16, half the output bytes), scales
    packed by pack_mxfp4_scales (k % 256 == 0)."""
    torch = _torch()
    for t, nm in ((codes_a, "codes_a"), (packed_scales_a, "packed_scales_a"), (codes_w, "codes_w"),
                  (packed_scales_w, "packed_scales_w")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    m, kb = codes_a.shape
    n = codes_w.shape[0]
    k = kb * 2
    if tuple(codes_w.shape) != (n, kb) or packed_scales_a.numel() != m * (k // 32) or \
            packed_scales_w.numel() != n * (k // 32):
        raise ValueError("operand shapes do not match")
    odt = torch.bfloat16 if bf16 else torch.float32
    if out is None:
        out = torch.empty((m, n), dtype=odt, device=codes_a.device)
    _dev(out, "out", (odt,))
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError("out must be %s [m][n] with unit column stride" % ("bf16" if bf16 else "fp32"))
    name = "kq_mxfp4_gemm_packed_bf16" if bf16 else "kq_mxfp4_gemm_packed"
    _check(name, getattr(lib(), name)(_p(codes_a), _p(packed_scales_a), _p(codes_w), _p(packed_scales_w), m, n, k,
                                      _p(out), out.stride(0), _stream_ptr(stream)))
    return out


def mxfp4_gemm_packed_lowrank(codes_a, packed_scales_a, codes_w, packed_scales_w, Z, codes_l, scales_l, out=None,
                              stream=None):
    """O = deq(A) deq(W)^T + Z deq(L)^T on the packed-scale GEMM (k % 256 == 0): Z fp32 [m][r],
    L in MXFP4 (codes [n][r/2], scales [n][r/32])."""
    torch = _torch()
    for t, nm in ((codes_a, "codes_a"), (packed_scales_a, "packed_scales_a"), (codes_w, "codes_w"),
                  (packed_scales_w, "packed_scales_w"), (codes_l, "codes_l"), (scales_l, "scales_l")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    _dev(Z, "Z", (torch.float32,))
    m, kb = codes_a.shape
    n = codes_w.shape[0]
    k = kb * 2
    r = Z.shape[1] if Z.dim() == 2 else -1
    if tuple(codes_w.shape) != (n, kb) or packed_scales_a.numel() != m * (k // 32) or \
            packed_scales_w.numel() != n * (k // 32) or tuple(Z.shape) != (m, r) or not Z.is_contiguous() or \
            tuple(codes_l.shape) != (n, r // 2) or tuple(scales_l.shape) != (n, r // 32):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=codes_a.device)
    _dev(out, "out", (torch.float32,))
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError("out must be fp32 [m][n] with unit column stride")
    _check("kq_mxfp4_gemm_packed_lowrank",
           lib().kq_mxfp4_gemm_packed_lowrank(_p(codes_a), _p(packed_scales_a), _p(codes_w), _p(packed_scales_w), m,
                                              n, k, _p(Z), _p(codes_l), _p(scales_l), r, _p(out), out.stride(0),
                                              _stream_ptr(stream)))
    return out


def mxfp4_gemm_packed_lowrank_split(codes_a, packed_scales_a, codes_w, packed_scales_w, Zh, Zl, L16, out=None,
                                    stream=None):
    """mxfp4_gemm_packed_lowrank with the branch's operands prepared once: Z split as Zh, Zl
    (bf16 [m][r], lowrank_project_bf16_split) and deq(L) in bf16 [n][r]
    (dequantize_mxfp4_bf16 of L). Bit-identical to the fp32-Z form on the Z they split."""
    torch = _torch()
    for t, nm in ((codes_a, "codes_a"), (packed_scales_a, "packed_scales_a"), (codes_w, "codes_w"),
                  (packed_scales_w, "packed_scales_w")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    for t, nm in ((Zh, "Zh"), (Zl, "Zl"), (L16, "L16")):
        _dev(t, nm, (torch.bfloat16, torch.int16, torch.uint16))
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(nm + " must be a contiguous 2-d bf16 tensor")
    m, kb = codes_a.shape
    n = codes_w.shape[0]
    k = kb * 2
    r = Zh.shape[1]
    if tuple(codes_w.shape) != (n, kb) or packed_scales_a.numel() != m * (k // 32) or \
            packed_scales_w.numel() != n * (k // 32) or tuple(Zh.shape) != (m, r) or tuple(Zl.shape) != (m, r) or \
            tuple(L16.shape) != (n, r):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=codes_a.device)
    _dev(out, "out", (torch.float32,))
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError("out must be fp32 [m][n] with unit column stride")
    _check("kq_mxfp4_gemm_packed_lowrank_split",
           lib().kq_mxfp4_gemm_packed_lowrank_split(_p(codes_a), _p(packed_scales_a), _p(codes_w),
                                                    _p(packed_scales_w), m, n, k, _p(Zh), _p(Zl), _p(L16), r,
                                                    _p(out), out.stride(0), _stream_ptr(stream)))
    return out


def mxfp4_gemm_wide(codes_a, scales_a, codes_w, scales_w, out=None, stream=None):
    """As mxfp4_gemm, on the 128 x 512-tile kernel (bit-identical results)."""
    torch = _torch()
    m, n, k, out = _gemm_operands(codes_a, scales_a, codes_w, scales_w, out)
    _check("kq_mxfp4_gemm_wide",
           lib().kq_mxfp4_gemm_wide(_p(codes_a), _p(scales_a), _p(codes_w), _p(scales_w), m, n, k, _p(out),
                                    out.stride(0), _stream_ptr(stream)))
    return out


def transform_quantize_mxfp4_gemm(A, factors, codes_w, scales_w, out=None, stream=None):
    """O = deq(Q(A T)) deq(W)^T in fp32: the Kronecker transform and MXFP4 quantizer of A
    (bf16 [m][k], factors fp32 [k/32][5][2][2]) run inside the W4A4 product with the MXFP4
    weights (codes [n][k/2], scales [n][k/32])."""
    torch = _torch()
    m, k, lda = _bf16_input(A)
    _dev(factors, "factors", (torch.float32,))
    if factors.numel() != (k // 32) * 20 or not factors.is_contiguous():
        raise ValueError("factors must be contiguous fp32 [k/32][5][2][2]")
    for t, nm in ((codes_w, "codes_w"), (scales_w, "scales_w")):
        _dev(t, nm, (torch.uint8,))
        if not t.is_contiguous():
            raise ValueError(nm + " must be contiguous")
    n = codes_w.shape[0]
    if tuple(codes_w.shape) != (n, k // 2) or tuple(scales_w.shape) != (n, k // 32):
        raise ValueError("weight operand shapes do not match A")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=A.device)
    _dev(out, "out", (torch.float32,))
    if out.dim() != 2 or out.shape[0] != m or out.shape[1] != n or out.stride(1) != 1:
        raise ValueError("out must be fp32 [m][n] with unit column stride")
    _check("kq_transform_quantize_mxfp4_gemm",
           lib().kq_transform_quantize_mxfp4_gemm(_p(A), m, k, lda, _p(factors), _p(codes_w), _p(scales_w), n,
                                                  _p(out), out.stride(0), _stream_ptr(stream)))
    return out


def gemm_f32(A, B, transa=False, transb=False, alpha=1.0, beta=0.0, C=None, out=None, stream=None):
    """D = alpha op(A) op(B) + beta C in fp32 (row-major operands)."""
    torch = _torch()
    for t, nm in ((A, "A"), (B, "B")):
        _dev(t, nm, (torch.float32,))
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(nm + " must be 2-D with unit column stride")
    m, k = (A.shape[1], A.shape[0]) if transa else (A.shape[0], A.shape[1])
    kb, n = (B.shape[1], B.shape[0]) if transb else (B.shape[0], B.shape[1])
    if kb != k:
        raise ValueError("inner dimensions do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=A.device)
    _dev(out, "out", (torch.float32,))
    if tuple(out.shape) != (m, n) or out.stride(1) != 1:
        raise ValueError("out must be fp32 [m][n] with unit column stride")
    if beta != 0.0:
        _dev(C, "C", (torch.float32,))
        if tuple(C.shape) != (m, n) or C.stride(1) != 1 or C.stride(0) != out.stride(0):
            raise ValueError("C must be fp32 [m][n] with the row stride of out")
    _check("kq_gemm_f32",
           lib().kq_gemm_f32(int(transa), int(transb), m, n, k, float(alpha), _p(A), A.stride(0), _p(B),
                             B.stride(0), float(beta), _p(C) if beta != 0.0 else None, out.stride(0), _p(out),
                             out.stride(0), _stream_ptr(stream)))
    return out


class Calibration:
    """Layer-wise calibration of the Kronecker factors (Sec. 3.3) on one GPU.

    Holds the device state: the 15 parameters per block (a, b, c of Eq. 6 for
    each of the five factors), Adam's moments, the Eq. 10 weights and the
    workspace. Every computation runs in libkq.so (kq_calib_init / kq_calib_step).
    """

    def __init__(self, A, W, theta=None, stream=None):
        torch = _torch()
        _dev(A, "A", (torch.bfloat16, torch.int16, torch.uint16))
        _dev(W, "W", (torch.float32,))
        if not A.is_contiguous() or not W.is_contiguous() or A.dim() != 2 or W.dim() != 2:
            raise ValueError("A [M][d] and W [o][d] must be contiguous")
        self.M, self.d = A.shape
        self.o = W.shape[0]
        if W.shape[1] != self.d:
            raise ValueError("W must be [o][d]")
        self.W = W
        self.stream = stream
        nbytes = ctypes.c_int64(0)
        _check("kq_calib_workspace_bytes",
               lib().kq_calib_workspace_bytes(self.M, self.d, self.o, ctypes.byref(nbytes)))
        self.ws = torch.empty(nbytes.value + 256, dtype=torch.uint8, device=A.device)
        self._ws_ptr = (self.ws.data_ptr() + 255) // 256 * 256
        nblk = self.d // 32
        if theta is None:  # Hadamard initialization (Sec. 3.2): a = b = 1/sqrt(2), c = 1
            theta = torch.tensor([2.0 ** -0.5, 2.0 ** -0.5, 1.0], dtype=torch.float32).repeat(nblk, 5, 1)
        self.theta = theta.to(device=A.device, dtype=torch.float32).contiguous().clone()
        if self.theta.numel() != nblk * 15:
            raise ValueError("theta must hold 15 parameters per block")
        self.m = torch.zeros_like(self.theta)
        self.v = torch.zeros_like(self.theta)
        self.lambdas = torch.zeros(2, dtype=torch.float32, device=A.device)
        self.losses = torch.zeros(3, dtype=torch.float32, device=A.device)
        self.grad = torch.zeros_like(self.theta)
        self.t = 0
        _check("kq_calib_init",
               lib().kq_calib_init(_p(A), self.M, self.d, _p(W), self.o, ctypes.c_void_p(self._ws_ptr),
                                   self.ws.numel() - 256, _stream_ptr(stream)))

    def step(self, lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, auto_lambda=None):
        """One Adam step (App. D.1: 100 steps at learning rate 1e-2); the first step (at
        the starting point) sets lambda by Eq. 10 unless ``auto_lambda`` is False (then
        ``self.lambdas`` is used as set)."""
        self.t += 1
        auto = (self.t == 1) if auto_lambda is None else bool(auto_lambda)
        _check("kq_calib_step",
               lib().kq_calib_step(_p(self.W), self.M, self.d, self.o, _p(self.theta), _p(self.m), _p(self.v),
                                   self.t, float(lr), float(beta1), float(beta2), float(eps), _p(self.lambdas),
                                   int(auto), _p(self.losses), _p(self.grad), ctypes.c_void_p(self._ws_ptr),
                                   self.ws.numel() - 256, _stream_ptr(self.stream)))
        return self.losses

    def factors(self):
        """The current 2x2 factors, fp32 [d/32][5][2][2] (Eq. 6), for the fused quantizer."""
        return factors_from_lu(self.theta.double().cpu().numpy())


def calib_step_noalloc(A, W, theta, adam_m, adam_v, t, lambdas, losses, grad=None, lr=1e-2, beta1=0.9,
                       beta2=0.999, eps=1e-8, auto_lambda=False, stream=None):
    """One calibration step (kq_calib_init + kq_calib_step) on the library's own
    device workspace (kq_calib_step_noalloc): nothing is allocated. theta, adam_m,
    adam_v, lambdas and losses are updated in place, as by Calibration.step."""
    torch = _torch()
    _dev(A, "A", (torch.bfloat16, torch.int16, torch.uint16))
    _dev(W, "W", (torch.float32,))
    M, d = A.shape
    o = W.shape[0]
    for name, x in (("theta", theta), ("adam_m", adam_m), ("adam_v", adam_v), ("lambdas", lambdas),
                    ("losses", losses)):
        _dev(x, name, (torch.float32,))
    _check("kq_calib_step_noalloc",
           lib().kq_calib_step_noalloc(_p(A), _p(W), M, d, o, _p(theta), _p(adam_m), _p(adam_v), int(t), float(lr),
                                       float(beta1), float(beta2), float(eps), _p(lambdas), int(bool(auto_lambda)),
                                       _p(losses), _p(grad) if grad is not None else None, _stream_ptr(stream)))
    return losses


def factors_from_lu(abc):
    """Host helper: (a, b, c) per factor, fp64 [nblk][5][3] -> fp32 [nblk][5][2][2] (Eq. 6)."""
    abc = np.ascontiguousarray(abc, dtype=np.float64)
    nblk = abc.shape[0]
    out = np.empty((nblk, 5, 2, 2), dtype=np.float32)
    _check("kq_factors_from_lu",
           lib().kq_factors_from_lu(ctypes.c_void_p(abc.ctypes.data), nblk,
                                    ctypes.c_void_p(out.ctypes.data)))
    return out
