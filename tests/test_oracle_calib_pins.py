"""Pins of the calibration oracle (oracle/calib.py; KroQuant Sec. 3.3, Eq. 6-10), no GPU.

- Eq. 6 and the Hadamard initialization against the closed form and the C
  oracle's independent Eq. 6 routine;
- the forward pass (A T and W T^{-T}) against the C oracle's transform and fold,
  and Eq. 1's invariance without quantization;
- the straight-through gradient against central finite differences of the
  surrogate it is the exact gradient of: the loss with the quantization
  residuals Q(X) - X, Q(Y) - Y frozen at the current point (and Q held fixed
  inside Eq. 8);
- Eq. 10's weights, and Adam's first steps against its closed form.
"""
import numpy as np
import pytest

import synth
from oracle import calib


def small_problem(orc, seed=3, M=96, d=64, o=40):
    z = synth.normal(synth.stream_key(seed, 0), 0, M * d).reshape(M, d)
    z[:, 5] *= 30.0  # an outlier channel, as in the paper's activations
    A = synth.bf16_bits_to_f32(synth.to_bf16_bits(z)).astype(np.float64)  # exact bf16 values
    W = synth.weights(o, d, seed + 1).astype(np.float64)
    return calib.Problem(A, W, orc)


def perturbed_theta(nblk, seed):
    rng = np.random.default_rng(seed)
    th = calib.hadamard_theta(nblk)
    return th + 0.05 * rng.standard_normal(th.shape)


def test_hadamard_init_is_sylvester(orc):
    G = calib.factors(calib.hadamard_theta(3))
    h = np.array([[1.0, 1.0], [1.0, -1.0]]) / np.sqrt(2.0)
    assert np.allclose(G, h, atol=1e-15)
    K = calib.kron5(G[0])
    r = np.arange(32)[:, None] & np.arange(32)[None, :]
    par = np.vectorize(lambda v: bin(v).count("1") & 1)(r)
    assert np.allclose(K, np.where(par == 1, -1.0, 1.0) / np.sqrt(32.0), atol=1e-15)


def test_eq6_matches_c_oracle(orc):
    th = perturbed_theta(4, 1)
    assert np.allclose(calib.factors(th), orc.factors_from_lu(th), rtol=0, atol=1e-15)


def test_forward_matches_c_transform_and_fold(orc):
    P = small_problem(orc)
    th = perturbed_theta(P.d // 32, 2)
    f = P.forward(th)
    fac32 = calib.factors(th).astype(np.float32)
    A_bits = synth.to_bf16_bits(P.A)
    Xc = orc.transform(A_bits, fac32)
    Yc = orc.inverse_fold(P.W.astype(np.float32), fac32)
    sx = np.abs(P.A).reshape(P.M, -1, 32).sum(axis=2).repeat(32, axis=1)
    assert (np.abs(f["X"] - Xc) <= 1e-6 * sx).all()
    assert np.allclose(f["Y"], Yc, rtol=1e-5, atol=1e-6 * np.abs(P.W).max())
    # Eq. 1 without quantization: (A T)(W T^{-T})^T = A W^T
    assert np.allclose(f["X"] @ f["Y"].T, P.C0, rtol=0, atol=1e-10 * np.abs(P.C0).max())


def surrogate(P, theta, frozen, lam_A, lam_W):
    """The loss with the quantization residuals and the Eq. 8 targets frozen at `frozen`."""
    f = P.forward(theta)
    rX, rY = frozen["Xq"] - frozen["X"], frozen["Yq"] - frozen["Y"]
    E = (f["X"] + rX) @ (f["Y"] + rY).T - P.C0
    return (E ** 2).sum() / (P.M * P.o) + \
        lam_A * ((frozen["Xq"] - f["X"]) ** 2).sum() / (P.M * P.d) + \
        lam_W * ((frozen["Yq"] - f["Y"]) ** 2).sum() / (P.o * P.d)


def check_gradient(orc, cal, seed):
    """The analytic gradient of module `cal` against finite differences of its own forward pass."""
    base = small_problem(orc, seed=seed)
    P = cal.Problem(base.A, base.W, orc)
    nblk = P.d // 32
    th = perturbed_theta(nblk, seed)
    lam_A, lam_W = 0.7, 1.9
    g = P.gradient(th, lam_A, lam_W)["dtheta"]
    frozen = P.forward(th)
    assert abs(surrogate(P, th, frozen, lam_A, lam_W) -
               P.gradient(th, lam_A, lam_W)["L"]) < 1e-12  # the surrogate equals L at the point
    h = 1e-6
    fd = np.empty_like(th)
    for idx in np.ndindex(th.shape):
        tp, tm = th.copy(), th.copy()
        tp[idx] += h
        tm[idx] -= h
        fd[idx] = (surrogate(P, tp, frozen, lam_A, lam_W) - surrogate(P, tm, frozen, lam_A, lam_W)) / (2 * h)
    assert np.allclose(g, fd, rtol=1e-5, atol=1e-7 * np.abs(fd).max())


@pytest.mark.parametrize("seed", [2, 7])
def test_ste_gradient_matches_finite_differences(orc, seed):
    check_gradient(orc, calib, seed)


def test_lambdas_balance_terms_at_init(orc):
    P = small_problem(orc)
    th0 = calib.hadamard_theta(P.d // 32)
    lam_A, lam_W = P.lambdas(th0)
    f = P.forward(th0)
    assert np.isclose(lam_A * f["L_A"], f["L_out"]) and np.isclose(lam_W * f["L_W"], f["L_out"])


def test_adam_closed_form():
    rng = np.random.default_rng(4)
    th = rng.standard_normal((2, 5, 3))
    g1, g2 = rng.standard_normal((2,) + th.shape)
    m = v = np.zeros_like(th)
    lr, b1, b2 = 1e-2, 0.9, 0.999
    t1, m, v = calib.adam_step(th, g1, m, v, 1, lr, b1, b2, eps=0.0)
    assert np.allclose(t1, th - lr * np.sign(g1), rtol=0, atol=1e-15)  # first step: -lr sign(g)
    t2, m, v = calib.adam_step(t1, g2, m, v, 2, lr, b1, b2, eps=0.0)
    # Kingma and Ba's step-size form: alpha_t = lr sqrt(1 - b2^t) / (1 - b1^t), theta -= alpha_t m / sqrt(v)
    mm = b1 * (1 - b1) * g1 + (1 - b1) * g2
    vv = b2 * (1 - b2) * g1 ** 2 + (1 - b2) * g2 ** 2
    alpha = lr * np.sqrt(1 - b2 ** 2) / (1 - b1 ** 2)
    assert np.allclose(t2, t1 - alpha * mm / np.sqrt(vv), rtol=1e-12, atol=1e-14)
