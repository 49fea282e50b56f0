"""The W4A4 layer with a low-rank branch -- CPU ORACLE (test infrastructure only).

KroQuant (arXiv 2607.21446v1) Sec. 3.4, Eq. 11: at inference a layer computes
    O = Q(A T) Q(W~ - L R)^T + (A T) R^T L^T,
W~ = W T^{-T} (Eq. 1), L (o x r) and R (r x d) the low-rank branch. App. D: the
activations entering the low-rank branch stay 16-bit and L, R are stored in
MXFP4 (rank 128). Readings taken where the pages are silent:
  - the branch's activation is A T rounded once to bf16 (nearest, ties to even);
  - Z = bf16(A T) Q(R)^T is kept at full precision (fp32 on the GPU, float64
    here), then O_lr = Z Q(L)^T;
  - Q is the MXFP4 quantizer of the C oracle, blocks of 32 along the contraction
    dimension (d for R and for the residual weights, r for L).
Float64 throughout except the one bf16 rounding. Only the tests, the smoke
check and the bench's CPU leg use this module.
"""
from __future__ import annotations

import numpy as np

from . import get as _get_oracle


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), as float64; finite inputs."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: round m * 2^8 to an integer, ties to even
    scaled = m * 256.0
    r = np.round(scaled)                     # numpy rounds half to even
    out = np.ldexp(r / 256.0, e)
    # below the smallest normal bf16 (2^-126) the grid is 2^-133
    tiny = np.abs(x) < 2.0 ** -126
    out[tiny] = np.round(x[tiny] * 2.0 ** 133) * 2.0 ** -133
    return out


def qdq(X: np.ndarray, orc=None) -> np.ndarray:
    orc = orc or _get_oracle()
    codes, scales = orc.quantize_f64(X)
    return orc.dequantize(codes, scales, X.shape[1])


def layer(A_bits, W, factors, L, R, orc=None, quantize=True):
    """Eq. 11 for bf16 activations A_bits [M][d], weights W [o][d], fp32 factors
    [d/32][5][2][2], L [o][r], R [r][d]. ``quantize=False`` replaces Q (and the
    bf16 rounding) by the identity. Returns (O, parts) with the two terms."""
    orc = orc or _get_oracle()
    X = orc.transform(A_bits, factors)                         # A T
    Wt = orc.inverse_fold(np.asarray(W, dtype=np.float32), factors)  # W T^{-T}
    L = np.asarray(L, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    resid = Wt - L @ R
    if quantize:
        main = qdq(X, orc) @ qdq(resid, orc).T
        Z = round_bf16(X) @ qdq(R, orc).T
        low = Z @ qdq(L, orc).T
    else:
        main = X @ resid.T
        Z = X @ R.T
        low = Z @ L.T
    return main + low, dict(main=main, low=low, Z=Z)
