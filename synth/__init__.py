"""Seeded synthetic inputs for the KroQuant activation quantizer.

This module is shared by the tests, the bench and the smoke check. It draws
activations, per-block Kronecker factors, weights and the SmoothQuant scale
vector; it holds none of the quantizer's or the transform's arithmetic, and it
imports neither the oracle nor the GPU package.

Random numbers come from one counter-based generator, SplitMix64 (Steele, Lea
and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the
n-th output of a stream keyed by ``k`` is ``mix64(k + (n + 1) * GAMMA)``, so any
element can be drawn independently of the others and the result does not
depend on chunking. Uniforms take the top 53 bits; normals use the Box-Muller
transform (cosine branch) on two consecutive uniforms. Values are rounded from
float64 straight to bfloat16 with round-to-nearest-even (no detour via fp32).

The shapes and distributions stand in for the DiT activations the KroQuant
paper (arXiv 2607.21446, Sec. 4.4 and Appendix A, Tables 3-4) times on: its
PixArt-Sigma and FLUX.1-schnell linear-layer inputs, which are not available
here. Factors follow the paper's Sec. 3.2 (2x2 factors of unit |det|, with the
normalized 2x2 Hadamard as the initialization).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

# Sub-stream identifiers (one SplitMix64 key per role and seed).
S_Z, S_SIGMA, S_TOKEN, S_OUTLIER, S_SKEW, S_FACTOR, S_WEIGHT = range(7)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so next to it (gcc, plain C11)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC",
                               "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64, u64]
        lib.synth_uniform.argtypes = [u64, u64, i64, p]
        lib.synth_normal.argtypes = [u64, u64, i64, p]
        lib.synth_to_bf16.argtypes = [p, i64, p]
        lib.synth_activation.argtypes = [p, i64, i64, u64, p, p, p, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


def stream_key(seed: int, stream: int) -> int:
    """Key of sub-stream ``stream``: SplitMix64 output number ``stream`` seeded by ``seed``."""
    return int(_load().synth_stream_key(seed & 0xFFFFFFFFFFFFFFFF, stream))


def uniform(key: int, start: int, n: int) -> np.ndarray:
    """U[0,1) doubles number start..start+n-1 of the stream keyed by ``key``."""
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform(key, start, n, _ptr(out))
    return out


def normal(key: int, start: int, n: int) -> np.ndarray:
    """N(0,1) doubles number start..start+n-1 (Box-Muller on uniforms 2i, 2i+1)."""
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal(key, start, n, _ptr(out))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round-to-nearest-even), return uint16 bits.

    Rounds the float64 significand directly, so there is no double rounding
    through fp32. Inputs must be finite and inside the bf16 range.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Kronecker factors (paper Sec. 3.2, Eq. 5-6 and "Hadamard initialization")
# ---------------------------------------------------------------------------

H2 = np.array([[1.0, 1.0], [1.0, -1.0]]) / math.sqrt(2.0)


def hadamard_factors(nblk: int) -> np.ndarray:
    """All five factors of every block equal to the normalized 2x2 Hadamard, as fp32.

    Layout [nblk][5][2][2]; index 0 is G1 (the factor on the most significant
    channel bit), entry [row][col].
    """
    return np.broadcast_to(H2.astype(np.float32), (nblk, 5, 2, 2)).copy()


def lu_perturbed_factors(nblk: int, seed: int, sigma_ab: float = 0.3,
                         sigma_log_s: float = 0.2) -> np.ndarray:
    """Per-block, per-factor G = H2 . [[1,0],[a,1]] . [[s,b],[0,1/s]] (row-vector convention).

    a, b ~ N(0, sigma_ab), s = exp(N(0, sigma_log_s)); computed in float64 and
    rounded to fp32. |det G| = 1 up to that rounding.
    """
    key = stream_key(seed, S_FACTOR)
    z = normal(key, 0, nblk * 5 * 3).reshape(nblk, 5, 3)
    a = sigma_ab * z[..., 0]
    b = sigma_ab * z[..., 1]
    s = np.exp(sigma_log_s * z[..., 2])
    L = np.zeros((nblk, 5, 2, 2))
    L[..., 0, 0] = 1.0
    L[..., 1, 0] = a
    L[..., 1, 1] = 1.0
    U = np.zeros((nblk, 5, 2, 2))
    U[..., 0, 0] = s
    U[..., 0, 1] = b
    U[..., 1, 1] = 1.0 / s
    G = np.einsum("ij,bkjl,bklm->bkim", H2, L, U)
    return G.astype(np.float32)


def special_factors(nblk: int, kind: str) -> np.ndarray:
    """Factors whose product K maps bf16 inputs to exactly representable outputs.

    kind: 'identity', 'swap' ([[0,1],[1,0]]), 'signflip' (diag(1,-1)),
    'pow2' (diag(2, 1/2)), or 'mixed' (a fixed cycle of the four).
    """
    table = {
        "identity": [[1.0, 0.0], [0.0, 1.0]],
        "swap": [[0.0, 1.0], [1.0, 0.0]],
        "signflip": [[1.0, 0.0], [0.0, -1.0]],
        "pow2": [[2.0, 0.0], [0.0, 0.5]],
    }
    if kind == "mixed":
        order = ["swap", "signflip", "pow2", "identity", "swap"]
        one = np.array([table[k] for k in order], dtype=np.float32)
        return np.broadcast_to(one, (nblk, 5, 2, 2)).copy()
    g = np.array(table[kind], dtype=np.float32)
    return np.broadcast_to(g, (nblk, 5, 2, 2)).copy()


# ---------------------------------------------------------------------------
# Activations
# ---------------------------------------------------------------------------

def _pick_channels(key: int, d: int, count: int, offset: int = 0) -> np.ndarray:
    """``count`` distinct channels chosen by sorting seeded uniform keys."""
    u = uniform(key, offset, d)
    return np.sort(np.argsort(u, kind="stable")[:count])


@dataclass
class ActivationRecipe:
    """Distribution of x_ic = t_i * sigma_c * o_c * z_ic, rounded to bf16."""
    m: int
    d: int
    seed: int
    token_scale: tuple = (0.5, 2.0)        # t_i ~ U(lo, hi); None -> 1
    lognormal_sigma: float | None = 0.5    # sigma_c ~ LogNormal(0, s); None -> 1
    outlier_frac: float = 0.01             # fraction of outlier channels
    outlier_mult: tuple = (50.0, 100.0)    # o_c ~ U(lo, hi) (lo == hi: fixed)
    skew_frac: float = 0.0                 # channels with z = |N(0,1)| - 0.2
    fixed_outliers: tuple = ()             # explicit (channel, multiplier) pairs
    extra: dict = field(default_factory=dict)

    def channel_params(self):
        d = self.d
        sig = np.ones(d)
        if self.lognormal_sigma is not None:
            sig = np.exp(self.lognormal_sigma *
                         normal(stream_key(self.seed, S_SIGMA), 0, d))
        mult = np.ones(d)
        if self.outlier_frac > 0:
            k3 = stream_key(self.seed, S_OUTLIER)
            n_out = int(round(self.outlier_frac * d))
            ch = _pick_channels(k3, d, n_out)
            lo, hi = self.outlier_mult
            u = uniform(k3, d, d)
            mult[ch] = lo + (hi - lo) * u[ch]
        for c, v in self.fixed_outliers:
            mult[c] = v
        skew = np.zeros(d, dtype=bool)
        if self.skew_frac > 0:
            n_sk = int(round(self.skew_frac * d))
            skew[_pick_channels(stream_key(self.seed, S_SKEW), d, n_sk)] = True
        return sig * mult, skew

    def generate(self, nthreads: int | None = None) -> np.ndarray:
        """Returns A as a C-contiguous uint16 array [m][d] of bf16 bit patterns."""
        m, d = self.m, self.d
        colscale, skew = self.channel_params()
        kz = stream_key(self.seed, S_Z)
        tok = None
        if self.token_scale is not None:
            lo, hi = self.token_scale
            tok = lo + (hi - lo) * uniform(stream_key(self.seed, S_TOKEN), 0, m)
        out = np.empty((m, d), dtype=np.uint16)
        colscale = np.ascontiguousarray(colscale, dtype=np.float64)
        skew_u8 = np.ascontiguousarray(skew, dtype=np.uint8) if skew.any() else None
        _load().synth_activation(_ptr(out), m, d, kz, _ptr(tok), _ptr(colscale),
                                 _ptr(skew_u8), nthreads or host_threads())
        return out


def weights(o: int, d: int, seed: int) -> np.ndarray:
    """W in fp32, [o][d], entries N(0, 1/d)."""
    key = stream_key(seed, S_WEIGHT)
    w = normal(key, 0, o * d).reshape(o, d) / math.sqrt(d)
    return w.astype(np.float32)


def smoothquant_inv_scale(A_bits: np.ndarray, d: int | None = None) -> np.ndarray:
    """SmoothQuant calibration vector for alpha = 0.5, beta = 0 (paper Appendix D.2).

    gamma_c = sqrt(max_i |A_ic|) over all rows; returns fp32 1/gamma_c (computed
    in float64, then rounded once). An all-zero column gets 1.
    """
    if d is None:
        d = A_bits.shape[1]
    mag = (A_bits[:, :d] & np.uint16(0x7FFF))
    amax_bits = mag.max(axis=0)
    amax = bf16_bits_to_f32(amax_bits).astype(np.float64)
    inv = np.ones(d)
    nz = amax > 0
    inv[nz] = 1.0 / np.sqrt(amax[nz])
    return inv.astype(np.float32)


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    A: np.ndarray          # uint16 [m][d] bf16 bits
    factors: np.ndarray    # fp32 [d/32][5][2][2]
    inv_scale: np.ndarray  # fp32 [d]

    @property
    def m(self):
        return self.A.shape[0]

    @property
    def d(self):
        return self.A.shape[1]


WORKLOADS = {
    # Tiny case: 64x256, N(0,1) with channels 3 and 200 scaled x80, Hadamard factors.
    "tiny_64x256": dict(m=64, d=256, seed=1000, kind="tiny"),
    # PixArt-Sigma attention input: one 1024px image, 4096 tokens x 1152 channels.
    "pixart_attn_4096x1152": dict(m=4096, d=1152, seed=1001, kind="pixart"),
    # PixArt-Sigma FFN down-projection input (CFG batch 2 x 4096 tokens) x 4608.
    "pixart_ffn_8192x4608": dict(m=8192, d=4608, seed=1002, kind="ffn"),
    # FLUX.1-schnell: batch 4 x (4096 image + 512 text) tokens = 18432 rows.
    "flux_18432x3072": dict(m=18432, d=3072, seed=1003, kind="pixart"),
    "flux_18432x12288": dict(m=18432, d=12288, seed=1013, kind="pixart"),
    # Power-of-two widths of the paper's kernel-latency table (Sec. 4.4, Table 3),
    # where the full-width Walsh-Hadamard transform applies without padding.
    "pow2_4096x1024": dict(m=4096, d=1024, seed=1021, kind="pixart"),
    "pow2_4096x4096": dict(m=4096, d=4096, seed=1022, kind="pixart"),
    "pow2_4096x16384": dict(m=4096, d=16384, seed=1023, kind="pixart"),
    "pow2_512x4096": dict(m=512, d=4096, seed=1024, kind="pixart"),
    "pow2_512x16384": dict(m=512, d=16384, seed=1025, kind="pixart"),
    # Production linear-layer shapes of FLUX.1 and PixArt-Sigma the paper times
    # (Appendix A, Table 4); 4096x1152 is the PixArt attention input above.
    "prod_512x3072": dict(m=512, d=3072, seed=1031, kind="pixart"),
    "prod_512x12288": dict(m=512, d=12288, seed=1032, kind="pixart"),
    "prod_4096x3072": dict(m=4096, d=3072, seed=1033, kind="pixart"),
    "prod_4096x3456": dict(m=4096, d=3456, seed=1034, kind="pixart"),
    "prod_4096x4608": dict(m=4096, d=4608, seed=1035, kind="pixart"),
    "prod_4096x12288": dict(m=4096, d=12288, seed=1036, kind="pixart"),
}


def recipe(name: str, m: int | None = None) -> ActivationRecipe:
    spec = WORKLOADS[name]
    mm = spec["m"] if m is None else m
    if spec["kind"] == "tiny":
        return ActivationRecipe(m=mm, d=spec["d"], seed=spec["seed"], token_scale=None,
                                lognormal_sigma=None, outlier_frac=0.0,
                                fixed_outliers=((3, 80.0), (200, 80.0)))
    if spec["kind"] == "ffn":
        return ActivationRecipe(m=mm, d=spec["d"], seed=spec["seed"], outlier_frac=0.005,
                                outlier_mult=(100.0, 100.0), skew_frac=0.7)
    return ActivationRecipe(m=mm, d=spec["d"], seed=spec["seed"])


def workload(name: str, m: int | None = None) -> Workload:
    """Generate a named workload; ``m`` overrides the row count (same per-row law)."""
    spec = WORKLOADS[name]
    rec = recipe(name, m)
    A = rec.generate()
    nblk = rec.d // 32
    if spec["kind"] == "tiny":
        fac = hadamard_factors(nblk)
    else:
        fac = lu_perturbed_factors(nblk, spec["seed"])
    return Workload(name=name, A=A, factors=fac, inv_scale=smoothquant_inv_scale(A))


def random_bf16_matrix(m: int, d: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) activations in bf16 bits (for edge-case tests)."""
    z = normal(stream_key(seed, S_Z), 0, m * d).reshape(m, d)
    return to_bf16_bits(scale * z)
