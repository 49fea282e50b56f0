"""Layer-wise calibration of the Kronecker factors -- CPU ORACLE (test infrastructure only).

Plain float64 numpy, step by step as KroQuant (arXiv 2607.21446v1) Sec. 3.3
states it; only the tests, ``__graft_entry__.smoke()`` and the bench's
CPU-baseline leg use it. The quantizer is the C oracle's (``quantize_f64`` and
``dequantize``); everything else is written out here.

- Parameters: per block and factor k = 1..5 the triple (a, b, c) of Eq. 6,
  G = [[1,0],[c,1]] . [[a,b],[0,-1/a]] = [[a, b], [c a, c b - 1/a]]
  (15 per block, Sec. 3.3 "Optimization").
- Initialization (Sec. 3.2 "Hadamard initialization"): every G equal to
  [[cos pi/4, sin pi/4], [sin pi/4, -cos pi/4]], i.e. a = b = 1/sqrt(2), c = 1.
- Transform (Eq. 1, 4, 5): X = A T with K^(j) = G1 (x) ... (x) G5 per block;
  weights Y = W T^{-T} with K^{-1} = G1^{-1} (x) ... (x) G5^{-1} (Sec. 3.2).
- Loss (Eq. 7-9), M = N m rows of calibration activations:
    L_out = ||Q(X) Q(Y)^T - A W^T||_F^2 / (M o),
    L_A   = ||Q(X) - X||_F^2 / (M d),      L_W = ||Q(Y) - Y||_F^2 / (o d),
    L     = L_out + lambda_A L_A + lambda_W L_W.
- Automatic weights (Eq. 10): lambda_A = L_out(T0) / L_A(T0),
  lambda_W = L_out(T0) / L_W(T0) at the Hadamard initialization T0.
- Gradient with a straight-through estimator (Sec. 3.3 "Optimization"). The
  reading taken: inside the output product Q passes gradients unchanged
  (dQ(x)/dx = 1); inside the operand terms of Eq. 8 the quantized value is held
  fixed, so d L_A / dX = -2 (Q(X) - X) / (M d). (With the identity inside Eq. 8
  as well, those terms would have zero gradient and could not do what Sec. 3.3
  says they are for.)
- Adam (Kingma and Ba 2014) on the 15 parameters per block.
"""
from __future__ import annotations

import numpy as np

from . import get as _get_oracle

INV_SQRT2 = 1.0 / np.sqrt(2.0)


def hadamard_theta(nblk: int) -> np.ndarray:
    """(a, b, c) of the Hadamard initialization, [nblk][5][3]."""
    th = np.empty((nblk, 5, 3))
    th[..., 0] = INV_SQRT2
    th[..., 1] = INV_SQRT2
    th[..., 2] = 1.0
    return th


def factors(theta: np.ndarray) -> np.ndarray:
    """Eq. 6: G = [[a, b], [c a, c b - 1/a]] for every block and factor, [nblk][5][2][2]."""
    a, b, c = theta[..., 0], theta[..., 1], theta[..., 2]
    G = np.empty(theta.shape[:-1] + (2, 2))
    G[..., 0, 0] = a
    G[..., 0, 1] = b
    G[..., 1, 0] = c * a
    G[..., 1, 1] = c * b - 1.0 / a
    return G


def kron5(G5: np.ndarray) -> np.ndarray:
    """Eq. 5: G1 (x) G2 (x) G3 (x) G4 (x) G5 for one block ([5][2][2] -> [32][32])."""
    K = G5[0]
    for k in range(1, 5):
        K = np.kron(K, G5[k])
    return K


def blocks(G: np.ndarray):
    """K^(j) and (K^(j))^{-1} (as the Kronecker product of the 2x2 inverses) for every block."""
    K = np.stack([kron5(g) for g in G])
    Ginv = np.linalg.inv(G)
    Kinv = np.stack([kron5(g) for g in Ginv])
    return K, Kinv


def _blockwise(X: np.ndarray, mats: np.ndarray) -> np.ndarray:
    """Row blocks of 32 channels times their own 32x32 matrix: out[:, 32j:32j+32] = X_j @ mats[j]."""
    m, d = X.shape
    Xb = X.reshape(m, d // 32, 32)
    return np.einsum("mjr,jrc->mjc", Xb, mats).reshape(m, d)


def qdq(X: np.ndarray, orc=None) -> np.ndarray:
    """Q(X): MXFP4 quantize (the C oracle) and decode back to float64."""
    orc = orc or _get_oracle()
    codes, scales = orc.quantize_f64(X)
    return orc.dequantize(codes, scales, X.shape[1])


class Problem:
    """One layer's calibration problem: activations A (bf16 values as float64) and weights W."""

    def __init__(self, A: np.ndarray, W: np.ndarray, orc=None):
        self.A = np.asarray(A, dtype=np.float64)
        self.W = np.asarray(W, dtype=np.float64)
        self.M, self.d = self.A.shape
        self.o = self.W.shape[0]
        self.C0 = self.A @ self.W.T  # A W^T, the full-precision layer output
        self.orc = orc or _get_oracle()

    def forward(self, theta: np.ndarray) -> dict:
        G = factors(theta)
        K, Kinv = blocks(G)
        X = _blockwise(self.A, K)                                   # A T
        Y = _blockwise(self.W, np.transpose(Kinv, (0, 2, 1)))      # W T^{-T}: block times (K^{-1})^T
        Xq, Yq = qdq(X, self.orc), qdq(Y, self.orc)
        E = Xq @ Yq.T - self.C0
        return dict(G=G, K=K, Kinv=Kinv, X=X, Y=Y, Xq=Xq, Yq=Yq, E=E,
                    L_out=float((E ** 2).sum() / (self.M * self.o)),
                    L_A=float(((Xq - X) ** 2).sum() / (self.M * self.d)),
                    L_W=float(((Yq - Y) ** 2).sum() / (self.o * self.d)))

    def lambdas(self, theta0: np.ndarray):
        """Eq. 10 at theta0."""
        f = self.forward(theta0)
        return f["L_out"] / f["L_A"], f["L_out"] / f["L_W"]

    def gradient(self, theta: np.ndarray, lam_A: float, lam_W: float):
        """Loss terms and dL/dtheta ([nblk][5][3]) under the STE reading above."""
        f = self.forward(theta)
        M, d, o = self.M, self.d, self.o
        GX = 2.0 / (M * o) * (f["E"] @ f["Yq"]) - lam_A * 2.0 / (M * d) * (f["Xq"] - f["X"])
        GY = 2.0 / (M * o) * (f["E"].T @ f["Xq"]) - lam_W * 2.0 / (o * d) * (f["Yq"] - f["Y"])
        nblk = d // 32
        Ab = self.A.reshape(M, nblk, 32)
        Wb = self.W.reshape(o, nblk, 32)
        # X_j = A_j K_j  ->  dL/dK_j = A_j^T GX_j
        dK = np.einsum("mjr,mjc->jrc", Ab, GX.reshape(M, nblk, 32))
        # Y_j = W_j P_j with P_j = K_j^{-T}: dL/dP_j = W_j^T GY_j, and dP = -K^{-T} dK^T K^{-T}
        dP = np.einsum("mjr,mjc->jrc", Wb, GY.reshape(o, nblk, 32))
        KinvT = np.transpose(f["Kinv"], (0, 2, 1))
        dK = dK - KinvT @ np.transpose(dP, (0, 2, 1)) @ KinvT
        dG = kron_factor_grads(f["G"], dK)
        L = f["L_out"] + lam_A * f["L_A"] + lam_W * f["L_W"]
        return dict(L=L, L_out=f["L_out"], L_A=f["L_A"], L_W=f["L_W"], dK=dK, dG=dG,
                    dtheta=theta_grad(theta, dG))


def kron_factor_grads(G: np.ndarray, dK: np.ndarray) -> np.ndarray:
    """dL/dG_k from dL/dK by Eq. 12: K[r][c] = prod_k G_k[bit_{5-k}(r)][bit_{5-k}(c)], so
    dL/dG_k[p][q] = sum over r, c with bit_{5-k}(r) = p, bit_{5-k}(c) = q of
    dL/dK[r][c] * prod_{i != k} G_i[bit_{5-i}(r)][bit_{5-i}(c)]."""
    nblk = G.shape[0]
    r = np.arange(32)[:, None]
    c = np.arange(32)[None, :]
    out = np.zeros((nblk, 5, 2, 2))
    bits = [((r >> (4 - k)) & 1, (c >> (4 - k)) & 1) for k in range(5)]
    for j in range(nblk):
        for k in range(5):
            prod = np.ones((32, 32))
            for i in range(5):
                if i != k:
                    prod = prod * G[j, i][bits[i][0], bits[i][1]]
            w = dK[j] * prod
            for p in range(2):
                for q in range(2):
                    out[j, k, p, q] = w[(bits[k][0] == p) & (bits[k][1] == q)].sum()
    return out


def theta_grad(theta: np.ndarray, dG: np.ndarray) -> np.ndarray:
    """Chain rule through Eq. 6: G00 = a, G01 = b, G10 = c a, G11 = c b - 1/a."""
    a, b, c = theta[..., 0], theta[..., 1], theta[..., 2]
    g00, g01, g10, g11 = dG[..., 0, 0], dG[..., 0, 1], dG[..., 1, 0], dG[..., 1, 1]
    out = np.empty_like(theta)
    out[..., 0] = g00 + c * g10 + g11 / (a * a)
    out[..., 1] = g01 + c * g11
    out[..., 2] = a * g10 + b * g11
    return out


def adam_step(theta, g, m, v, t, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8):
    """One Adam update (Kingma and Ba 2014, Algorithm 1); returns new theta, m, v."""
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    return theta - lr * mhat / (np.sqrt(vhat) + eps), m, v
