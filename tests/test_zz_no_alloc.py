"""GPU: the allocation-free calibration step (kq_calib_step_noalloc, the library's own
device workspace) against kq_calib_init + kq_calib_step on a caller-owned workspace
(Sec. 3.3, Eq. 6-10): the same kernels in the same order, so theta, Adam's moments,
the Eq. 10 weights, the three loss terms and the gradient agree bit for bit. Two calls
in a row on the same device, the second on a smaller problem, and a problem whose
workspace exceeds the array is refused before anything is launched."""
import sys

import numpy as np
import pytest

import synth

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


def problem(torch, M, d, o, seed):
    A = synth.ActivationRecipe(m=M, d=d, seed=seed).generate()
    W = synth.weights(o, d, seed + 1)
    Ad = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    return Ad, torch.from_numpy(W).cuda()


def reference_step(torch, kq, A, W):
    cal = kq.Calibration(A, W)
    cal.step(lr=1e-2)  # t = 1, lambda set by Eq. 10
    torch.cuda.synchronize()
    return cal


def noalloc_step(torch, kq, A, W):
    nblk = A.shape[1] // 32
    theta = torch.tensor([2.0 ** -0.5, 2.0 ** -0.5, 1.0], dtype=torch.float32).repeat(nblk, 5, 1).cuda()
    m = torch.zeros_like(theta)
    v = torch.zeros_like(theta)
    lam = torch.zeros(2, dtype=torch.float32, device="cuda")
    losses = torch.zeros(3, dtype=torch.float32, device="cuda")
    grad = torch.zeros_like(theta)
    kq.calib_step_noalloc(A, W, theta, m, v, 1, lam, losses, grad, lr=1e-2, auto_lambda=True)
    torch.cuda.synchronize()
    return theta, m, v, lam, losses, grad


def test_noalloc_step_matches_workspace_step(torch_dev, kq):
    torch = torch_dev
    for (M, d, o, seed) in ((1024, 1152, 1152, 51), (256, 256, 128, 52)):
        case("calib noalloc M=%d d=%d o=%d" % (M, d, o))
        A, W = problem(torch, M, d, o, seed)
        ref = reference_step(torch, kq, A, W)
        theta, m, v, lam, losses, grad = noalloc_step(torch, kq, A, W)
        assert torch.equal(losses, ref.losses), (losses, ref.losses)
        assert torch.equal(lam, ref.lambdas)
        assert torch.equal(grad, ref.grad)
        assert torch.equal(theta, ref.theta)
        assert torch.equal(m, ref.m) and torch.equal(v, ref.v)
        assert bool(torch.isfinite(losses).all()) and float(losses[0]) > 0


def test_noalloc_step_refuses_above_the_limit(torch_dev, kq):
    torch = torch_dev
    case("calib noalloc over the limit")
    A, W = problem(torch, 4096, 1152, 1152, 53)  # 126 MiB of workspace
    nblk = 1152 // 32
    z = torch.zeros((nblk, 5, 3), dtype=torch.float32, device="cuda")
    s = torch.zeros(3, dtype=torch.float32, device="cuda")
    with pytest.raises(kq.KQError) as e:
        kq.calib_step_noalloc(A, W, z.clone(), z.clone(), z.clone(), 1, s[:2].clone(), s.clone())
    assert e.value.status == kq.KQ_ERR_UNSUPPORTED
