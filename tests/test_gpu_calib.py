"""GPU parity of the calibration path (Sec. 3.3) against the float64 oracle
(oracle/calib.py), through the C ABI: the fp32 GEMM, the loss terms, the
straight-through gradient, Eq. 10's weights and Adam's update, and a short run
that lowers the loss from the Hadamard start.

Tolerances: the GPU computes in fp32 (GEMM sums in ascending k) and the oracle
in float64; a quantized element may land on the other side of a rounding tie,
which moves the loss and gradient by far less than the bars below.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import calib

pytestmark = pytest.mark.gpu


def case(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


@pytest.fixture(scope="module")
def kq():
    import mxfp4_activation_quantizer_amd as kq
    kq.lib()
    return kq


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("m,n,k", [(70, 45, 37), (128, 64, 256), (1, 1, 1), (200, 136, 100), (257, 129, 64)])
def test_gemm_f32(torch_dev, kq, ta, tb, m, n, k):
    torch = torch_dev
    case("gemm ta=%d tb=%d %dx%dx%d" % (ta, tb, m, n, k))
    rng = np.random.default_rng(m * 7 + n + k)
    A = rng.standard_normal((k, m) if ta else (m, k)).astype(np.float32)
    B = rng.standard_normal((n, k) if tb else (k, n)).astype(np.float32)
    C = rng.standard_normal((m, n)).astype(np.float32)
    d = lambda x: torch.from_numpy(x).cuda()
    out = kq.gemm_f32(d(A), d(B), bool(ta), bool(tb), alpha=0.75, beta=-1.25, C=d(C))
    torch.cuda.synchronize()
    opA = A.T.astype(np.float64) if ta else A.astype(np.float64)
    opB = B.T.astype(np.float64) if tb else B.astype(np.float64)
    ref = 0.75 * opA @ opB - 1.25 * C
    bound = 2.0 ** -22 * (k + 2) * (0.75 * np.abs(opA) @ np.abs(opB) + 1.25 * np.abs(C))
    assert (np.abs(out.cpu().numpy() - ref) <= bound).all()


def problem(seed, M, d, o):
    rec = synth.ActivationRecipe(m=M, d=d, seed=seed)
    A_bits = rec.generate()
    W = synth.weights(o, d, seed + 1)
    return A_bits, W


def gpu_calibration(torch, kq, A_bits, W, theta):
    A = torch.from_numpy(A_bits.view(np.int16)).cuda().view(torch.bfloat16)
    return kq.Calibration(A, torch.from_numpy(W).cuda(), theta=torch.from_numpy(theta.astype(np.float32)))


def oracle_problem(orc, A_bits, W):
    return calib.Problem(synth.bf16_bits_to_f32(A_bits).astype(np.float64), W.astype(np.float64), orc)


@pytest.mark.parametrize("M,d,o", [(256, 128, 96), (300, 96, 70)])
def test_loss_and_gradient_match_oracle(torch_dev, kq, orc, M, d, o):
    torch = torch_dev
    case("calib gradient M=%d d=%d o=%d" % (M, d, o))
    A_bits, W = problem(500 + M, M, d, o)
    rng = np.random.default_rng(M)
    th = (calib.hadamard_theta(d // 32) + 0.05 * rng.standard_normal((d // 32, 5, 3))).astype(np.float32)
    cal = gpu_calibration(torch, kq, A_bits, W, th)
    cal.lambdas.copy_(torch.tensor([0.7, 1.9]))
    cal.step(lr=0.0, auto_lambda=False)
    torch.cuda.synchronize()
    P = oracle_problem(orc, A_bits, W)
    ref = P.gradient(th.astype(np.float64), 0.7, 1.9)
    losses = cal.losses.cpu().numpy().astype(np.float64)
    got = dict(L_out=losses[0], L_A=losses[1], L_W=losses[2])
    for key in got:
        assert abs(got[key] - ref[key]) <= 2e-4 * abs(ref[key]), (key, got[key], ref[key])
    g = cal.grad.cpu().numpy().astype(np.float64)
    err = np.abs(g - ref["dtheta"]).max() / np.abs(ref["dtheta"]).max()
    print("[parity] calib M=%d d=%d o=%d: losses %s, grad max err / max |g| = %.2e" % (M, d, o, got, err),
          flush=True)
    assert err <= 2e-3
    # lr = 0 leaves theta unchanged
    assert np.array_equal(cal.theta.cpu().numpy(), th)


def test_auto_lambda_and_first_adam_step(torch_dev, kq, orc):
    torch = torch_dev
    case("calib lambda + adam")
    M, d, o = 256, 128, 96
    A_bits, W = problem(901, M, d, o)
    th0 = calib.hadamard_theta(d // 32)
    cal = gpu_calibration(torch, kq, A_bits, W, th0)
    lr = 1e-3
    cal.step(lr=lr)  # t = 1: sets lambda by Eq. 10, then updates
    torch.cuda.synchronize()
    P = oracle_problem(orc, A_bits, W)
    la, lw = P.lambdas(th0)
    lam = cal.lambdas.cpu().numpy()
    assert abs(lam[0] - la) <= 2e-4 * la and abs(lam[1] - lw) <= 2e-4 * lw
    g = P.gradient(th0, la, lw)["dtheta"]
    th1_ref, _, _ = calib.adam_step(th0, g, np.zeros_like(th0), np.zeros_like(th0), 1, lr=lr)
    th1 = cal.theta.cpu().numpy().astype(np.float64)
    big = np.abs(g) > 1e-2 * np.abs(g).max()  # the first step is lr * sign(g) wherever |g| >> eps
    assert np.allclose(th1[big], th1_ref[big], rtol=0, atol=1e-6)


def test_short_run_lowers_the_loss(torch_dev, kq):
    torch = torch_dev
    case("calib run")
    M, d, o = 512, 256, 192
    A_bits, W = problem(77, M, d, o)
    cal = gpu_calibration(torch, kq, A_bits, W, calib.hadamard_theta(d // 32))
    first = None
    for _ in range(60):
        losses = cal.step(lr=1e-2).cpu().numpy()
        first = losses.copy() if first is None else first
    last = cal.step(lr=0.0).cpu().numpy()
    print("[calib] L_out %.4f -> %.4f, L_A %.4f -> %.4f" % (first[0], last[0], first[1], last[1]), flush=True)
    assert last[0] < 0.5 * first[0]


def test_w4a4_calibrated_flux(torch_dev, kq, orc):
    """Calibrate on the first 4096 rows of the FLUX 18432x3072 activations with the
    3072x3072 weights, then run the whole W4A4 pipeline (fold, fp32 quantize, fused
    transform + quantize, MXFP4 GEMM) with the learned factors and compare the layer
    output error |Q(AT) Q(WT^-T)^T - A W^T| on held-out rows with T = I and with
    the block-Hadamard start. The pipeline itself is checked against the oracle's
    pipeline with the same learned factors."""
    torch = torch_dev
    case("w4a4 calibrated 18432x3072x3072")
    w = synth.workload("flux_18432x3072")
    W = synth.weights(3072, 3072, 1004)
    Wd = torch.from_numpy(W).cuda()
    A_dev = torch.from_numpy(w.A.view(np.int16)).cuda().view(torch.bfloat16)
    cal = kq.Calibration(A_dev[:4096].contiguous(), Wd)
    for _ in range(100):
        cal.step(lr=1e-2)
    losses = cal.step(lr=0.0).cpu().numpy()
    fac = torch.from_numpy(cal.factors()).cuda()

    def pipeline(f):
        if f is None:
            ca, sa = kq.quantize_mxfp4(A_dev)
            cw, sw = kq.quantize_mxfp4_f32(Wd)
        else:
            ca, sa = kq.transform_quantize_mxfp4(A_dev, f)
            cw, sw = kq.quantize_mxfp4_f32(kq.inverse_fold_weights(Wd, f))
        return kq.mxfp4_gemm(ca, sa, cw, sw)

    O_c = pipeline(fac)
    O_h = pipeline(torch.from_numpy(synth.hadamard_factors(96)).cuda())
    O_i = pipeline(None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(np.arange(4096, w.m), 256, replace=False))  # held out from calibration
    idx = torch.from_numpy(rows).cuda()
    exact = synth.bf16_bits_to_f32(w.A[rows]).astype(np.float64) @ W.astype(np.float64).T
    err = {k: np.linalg.norm(O.index_select(0, idx).cpu().numpy().astype(np.float64) - exact)
           for k, O in (("calibrated", O_c), ("hadamard", O_h), ("identity", O_i))}
    # the GPU pipeline with the learned factors against the oracle's pipeline (same factors)
    sub = rows[:64]
    facn = cal.factors()
    ca_r, sa_r, _ = orc.transform_quantize(w.A[sub], facn, want_y=False)
    cw_r, sw_r = orc.quantize_f64(orc.inverse_fold(W, facn))
    O_r = orc.gemm_dequant(ca_r, sa_r, cw_r, sw_r, 3072)
    og = O_c.index_select(0, torch.from_numpy(sub).cuda()).cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(og - O_r) / np.linalg.norm(O_r)
    print("[calib-w4a4] calibration losses %s; held-out |E|: calibrated %.1f, Hadamard %.1f, T=I %.1f; "
          "pipeline vs oracle %.2e" % (losses, err["calibrated"], err["hadamard"], err["identity"], rel), flush=True)
    assert rel <= 1e-3
    assert err["calibrated"] < err["hadamard"] and err["calibrated"] < err["identity"]
