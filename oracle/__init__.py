"""CPU oracle for the KroQuant activation quantizer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

The arithmetic lives in ``kq_oracle.c`` (plain C, float64, row-parallel with
pthreads); this module only compiles it with gcc and marshals numpy arrays.
What each function follows in the KroQuant paper (arXiv 2607.21446v1):

- ``quantize_*``: Sec. 3.1 blockwise quantizer with MXFP4 E2M1 elements and
  an E8M0 scale per 32-block (Sec. 4.1 "Data format", Appendix D), under the
  OCP MX conventions listed in the C file's header.
- ``block_K`` (Eq. 12), ``block_K_kron`` (Eq. 5), ``block_Kinv`` (Sec. 3.2:
  inverse of a Kronecker product is the product of the inverses).
- ``transform`` / ``transform_quantize``: Eq. 1's A -> A T with T from Eq. 4.
- ``smoothquant_quantize``: Appendix D.2 per-channel scaling, then quantize.
- ``inverse_fold``: Eq. 1's W -> W T^{-T}.
- ``gemm_dequant``: Eq. 2's Q(AT) Q(WT^{-T})^T in float64.
- ``factors_from_lu``: Eq. 6.
- ``hadamard_quantize`` / ``hadamard_f64``: the fixed block-Hadamard baselines
  (Sec. 1; Sec. 3.2 "Hadamard initialization" defines H_n; Sec. 4.4, Table 2's
  Hadamard-32 row and Table 3's full-width FWHT), then the same quantizer.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkq_oracle.so")
_lib = None

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-pthread", "-D_GNU_SOURCE"]


def build(force: bool = False, out: str | None = None, extra=()) -> str:
    """Compile kq_oracle.c with gcc into libkq_oracle.so (or ``out``)."""
    target = out or _LIB_PATH
    if force or out or not os.path.exists(target) or \
            os.path.getmtime(target) < os.path.getmtime(_SRC):
        tmp = target + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, *extra, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, target)
    return target


def _bind(lib):
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.kqo_bf16_to_double.restype = ctypes.c_double
    lib.kqo_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.kqo_e2m1_value.restype = ctypes.c_double
    lib.kqo_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.kqo_e2m1_round_index.restype = i32
    lib.kqo_e2m1_round_index.argtypes = [ctypes.c_double]
    lib.kqo_shared_exponent.restype = i32
    lib.kqo_shared_exponent.argtypes = [ctypes.c_double]
    lib.kqo_quantize_block.argtypes = [p, p, p]
    lib.kqo_block_K.argtypes = [p, p]
    lib.kqo_block_K_kron.argtypes = [p, p]
    lib.kqo_block_Kinv.argtypes = [p, p]
    lib.kqo_factors_from_lu.argtypes = [p, i64, p]
    lib.kqo_default_threads.restype = i32
    lib.kqo_quantize_bf16.argtypes = [p, i64, i64, i64, p, p, i32]
    lib.kqo_quantize_f32.argtypes = [p, i64, i64, i64, p, p, i32]
    lib.kqo_quantize_f64.argtypes = [p, i64, i64, i64, p, p, i32]
    lib.kqo_transform_quantize.restype = i32
    lib.kqo_transform_quantize.argtypes = [p, i64, i64, i64, p, p, p, p, i32]
    lib.kqo_smoothquant_quantize.argtypes = [p, i64, i64, i64, p, p, p, i32]
    lib.kqo_inverse_fold.restype = i32
    lib.kqo_inverse_fold.argtypes = [p, i64, i64, p, p, i32]
    lib.kqo_dequantize.argtypes = [p, p, i64, i64, p]
    lib.kqo_gemm_dequant.restype = i32
    lib.kqo_gemm_dequant.argtypes = [p, p, p, p, i64, i64, p, i64, p, i32]
    lib.kqo_hadamard_quantize.restype = i32
    lib.kqo_hadamard_quantize.argtypes = [p, i64, i64, i64, i64, p, p, p, i32]
    lib.kqo_hadamard_f64.restype = i32
    lib.kqo_hadamard_f64.argtypes = [p, i64, i64, i64, i64, p, i32]
    return lib


def load(path: str | None = None):
    """The oracle library (built on first use); ``path`` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return int(load().kqo_default_threads())


class Oracle:
    """Thin marshalling over one loaded build of the oracle library."""

    def __init__(self, lib=None, nthreads: int = 0):
        self.lib = lib or load()
        self.nthreads = nthreads

    # -- scalars -------------------------------------------------------------
    def e2m1_value(self, code: int) -> float:
        return self.lib.kqo_e2m1_value(code)

    def e2m1_round_index(self, v: float) -> int:
        return self.lib.kqo_e2m1_round_index(v)

    def shared_exponent(self, amax: float) -> int:
        return self.lib.kqo_shared_exponent(amax)

    def quantize_block(self, y):
        y = _c(y, np.float64)
        assert y.shape == (32,)
        codes = np.zeros(16, dtype=np.uint8)
        scale = np.zeros(1, dtype=np.uint8)
        self.lib.kqo_quantize_block(_p(y), _p(codes), _p(scale))
        return codes, int(scale[0])

    # -- Kronecker blocks ------------------------------------------------------
    def _blk(self, fn, factors20):
        f = _c(factors20, np.float32).reshape(20)
        K = np.empty((32, 32), dtype=np.float64)
        fn(_p(f), _p(K))
        return K

    def block_K(self, factors20):
        return self._blk(self.lib.kqo_block_K, factors20)

    def block_K_kron(self, factors20):
        return self._blk(self.lib.kqo_block_K_kron, factors20)

    def block_Kinv(self, factors20):
        return self._blk(self.lib.kqo_block_Kinv, factors20)

    def factors_from_lu(self, abc):
        abc = _c(abc, np.float64)
        nblk = abc.shape[0]
        G = np.empty((nblk, 5, 2, 2), dtype=np.float64)
        self.lib.kqo_factors_from_lu(_p(abc), nblk, _p(G))
        return G

    # -- the path ------------------------------------------------------------
    def _out(self, m, d):
        return (np.zeros((m, d // 2), dtype=np.uint8), np.zeros((m, d // 32), dtype=np.uint8))

    def quantize_bf16(self, A, d=None):
        A = _c(A, np.uint16)
        m, lda = A.shape
        d = lda if d is None else d
        codes, scales = self._out(m, d)
        self.lib.kqo_quantize_bf16(_p(A), m, d, lda, _p(codes), _p(scales), self.nthreads)
        return codes, scales

    def quantize_f32(self, X, d=None):
        X = _c(X, np.float32)
        m, ld = X.shape
        d = ld if d is None else d
        codes, scales = self._out(m, d)
        self.lib.kqo_quantize_f32(_p(X), m, d, ld, _p(codes), _p(scales), self.nthreads)
        return codes, scales

    def quantize_f64(self, Y, d=None):
        Y = _c(Y, np.float64)
        m, ld = Y.shape
        d = ld if d is None else d
        codes, scales = self._out(m, d)
        self.lib.kqo_quantize_f64(_p(Y), m, d, ld, _p(codes), _p(scales), self.nthreads)
        return codes, scales

    def transform_quantize(self, A, factors, d=None, want_y=True, want_codes=True):
        A = _c(A, np.uint16)
        f = _c(factors, np.float32)
        m, lda = A.shape
        d = lda if d is None else d
        assert f.size == (d // 32) * 20
        codes, scales = self._out(m, d) if want_codes else (None, None)
        y = np.empty((m, d), dtype=np.float64) if want_y else None
        rc = self.lib.kqo_transform_quantize(_p(A), m, d, lda, _p(f), _p(codes), _p(scales),
                                             _p(y), self.nthreads)
        if rc != 0:
            raise MemoryError("oracle transform")
        return codes, scales, y

    def transform(self, A, factors, d=None):
        return self.transform_quantize(A, factors, d, want_y=True, want_codes=False)[2]

    def smoothquant_quantize(self, A, inv_scale, d=None):
        A = _c(A, np.uint16)
        s = _c(inv_scale, np.float32)
        m, lda = A.shape
        d = lda if d is None else d
        codes, scales = self._out(m, d)
        self.lib.kqo_smoothquant_quantize(_p(A), m, d, lda, _p(s), _p(codes), _p(scales),
                                          self.nthreads)
        return codes, scales

    def inverse_fold(self, W, factors):
        W = _c(W, np.float32)
        f = _c(factors, np.float32)
        o, d = W.shape
        Wf = np.empty((o, d), dtype=np.float64)
        if self.lib.kqo_inverse_fold(_p(W), o, d, _p(f), _p(Wf), self.nthreads) != 0:
            raise MemoryError("oracle fold")
        return Wf

    def dequantize(self, codes, scales, d):
        codes = _c(codes, np.uint8)
        scales = _c(scales, np.uint8)
        m = codes.shape[0]
        out = np.empty((m, d), dtype=np.float64)
        self.lib.kqo_dequantize(_p(codes), _p(scales), m, d, _p(out))
        return out

    def gemm_dequant(self, codes_a, scales_a, codes_w, scales_w, k, rows=None):
        codes_a = _c(codes_a, np.uint8)
        scales_a = _c(scales_a, np.uint8)
        codes_w = _c(codes_w, np.uint8)
        scales_w = _c(scales_w, np.uint8)
        nout = codes_w.shape[0]
        rows = np.arange(codes_a.shape[0]) if rows is None else np.asarray(rows)
        rows = _c(rows, np.int64)
        O = np.empty((rows.size, nout), dtype=np.float64)
        rc = self.lib.kqo_gemm_dequant(_p(codes_a), _p(scales_a), _p(codes_w), _p(scales_w),
                                       nout, k, _p(rows), rows.size, _p(O), self.nthreads)
        if rc != 0:
            raise MemoryError("oracle gemm")
        return O

    def hadamard_quantize(self, A, n, d=None, want_y=True, want_codes=True):
        """Each group of n channels times H_n / sqrt(n), then MXFP4."""
        A = _c(A, np.uint16)
        m, lda = A.shape
        d = lda if d is None else d
        codes, scales = self._out(m, d) if want_codes else (None, None)
        y = np.empty((m, d), dtype=np.float64) if want_y else None
        rc = self.lib.kqo_hadamard_quantize(_p(A), m, d, lda, n, _p(codes), _p(scales), _p(y),
                                            self.nthreads)
        if rc != 0:
            raise ValueError("oracle hadamard: n must be a power of two dividing d")
        return codes, scales, y

    def hadamard_f64(self, X, n):
        X = _c(X, np.float64)
        m, d = X.shape
        y = np.empty((m, d), dtype=np.float64)
        if self.lib.kqo_hadamard_f64(_p(X), m, d, d, n, _p(y), self.nthreads) != 0:
            raise ValueError("oracle hadamard: n must be a power of two dividing d")
        return y


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
