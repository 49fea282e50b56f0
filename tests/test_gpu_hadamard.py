"""GPU parity of the block-Hadamard baseline (kq_hadamard_quantize_mxfp4)
against the oracle's dense Sylvester product, under the fused-path rules of
tests/parity.py (the transform runs in fp32 on the GPU, in float64 in the
oracle).

Group sizes n = 32 ... 16384 cover the Hadamard-32 baseline of the paper's
transform ablation (Table 2) and the full-width fast Walsh-Hadamard transform
of its kernel table (Sec. 4.4, Table 3), whose power-of-two shapes run here at
full size on sampled rows.
"""
import sys

import numpy as np
import pytest

import synth
from tests import parity

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


def dev_bf16(torch, A):
    return torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).to("cuda").view(torch.bfloat16)


def run(torch, kq, A_host, d, n, debug=True):
    """GPU codes, scales (and y) of A_host[:, :d] (A_host may be wider: padded rows)."""
    m = A_host.shape[0]
    A = dev_bf16(torch, A_host)[:, :d]
    y = torch.empty((m, d), dtype=torch.float32, device="cuda") if debug else None
    codes, scales = kq.hadamard_quantize_mxfp4(A, n, y_debug=y)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (y.cpu().numpy() if debug else None)


SMALL = [
    # (n, m, d, lda): every stage placement, ragged tiles, several groups per row, padded rows
    (32, 70, 96, 104), (32, 1, 32, 32), (64, 33, 128, 128), (128, 9, 384, 392), (256, 5, 512, 512),
    (256, 7, 768, 776), (512, 6, 1024, 1024), (512, 3, 1536, 1544), (1024, 4, 2048, 2048),
    (1024, 3, 3072, 3080), (2048, 3, 2048, 2056), (2048, 5, 6144, 6144), (4096, 3, 4096, 4096),
    (4096, 2, 8192, 8200), (8192, 3, 8192, 8192), (8192, 2, 16384, 16392), (16384, 2, 16384, 16384),
    (16384, 3, 16384, 16392), (16384, 1, 32768, 32768),
]


@pytest.mark.parametrize("n,m,d,lda", SMALL)
def test_hadamard_parity_small(torch_dev, kq, orc, n, m, d, lda):
    torch = torch_dev
    case("hadamard n=%d m=%d d=%d lda=%d" % (n, m, d, lda))
    A = synth.random_bf16_matrix(m, lda, seed=7 * n + m)
    A[:, d:] = 0x7FC0  # padding must never be read: NaN would poison a group
    codes, scales, y = run(torch, kq, A, d, n)
    _, _, yr = orc.hadamard_quantize(A, n, d=d, want_codes=False)
    rep = parity.fused_report(orc, A[:, :d], None, codes, scales, y, y_ref=yr)
    print("[parity] hadamard n=%d: %s" % (n, rep), flush=True)
    c2, s2, _ = run(torch, kq, A, d, n, debug=False)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales), "check mode changed the codes"


def test_hadamard32_worked_example(torch_dev, kq):
    """One bf16 80 at channel 3 of a block: y = +-80/sqrt(32) = +-14.14 -> scale byte 128,
    every |v| = 7.07 saturates to code 7 with the sign (-1)^popcount(3 & c)."""
    torch = torch_dev
    A = np.zeros((4, 64), dtype=np.uint16)
    A[:, 3] = synth.to_bf16_bits(np.array([80.0]))[0]
    codes, scales, _ = run(torch, kq, A, 64, 32)
    assert (scales[:, 0] == 128).all() and (scales[:, 1] == 0).all()
    nib = parity.unpack(codes)
    for c in range(32):
        want = 7 | (8 if bin(3 & c).count("1") & 1 else 0)
        assert (nib[:, c] == want).all(), c


@pytest.mark.parametrize("n", [1024, 16384])
def test_full_width_constant_row_exact(torch_dev, kq, n):
    """All ones: H_n 1 / sqrt(n) = sqrt(n) e_0 (exact in fp32 for n = 4^k). The zeros
    may come out as -0 (an exact zero times a negative sign), which the fused-path
    rule treats as +0."""
    torch = torch_dev
    A = np.full((3, n), 0x3F80, dtype=np.uint16)
    codes, scales, y = run(torch, kq, A, n, n)
    want = np.zeros(n, dtype=np.float32)
    want[0] = np.sqrt(n)
    assert np.array_equal(y, np.broadcast_to(want, y.shape))
    e = int(np.log2(np.sqrt(n))) - 2 + 127
    assert (scales[:, 0] == e).all() and (scales[:, 1:] == 0).all()
    nib = parity.zero_equiv(parity.unpack(codes))
    assert (nib[:, 0] == 6).all() and (nib[:, 1:] == 0).all()


def test_empty(torch_dev, kq):
    torch = torch_dev
    A = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    codes, scales = kq.hadamard_quantize_mxfp4(A, 1024)
    assert codes.shape == (0, 512) and scales.shape == (0, 32)


POW2 = ["pow2_4096x1024", "pow2_4096x4096", "pow2_4096x16384", "pow2_512x4096", "pow2_512x16384"]


@pytest.mark.parametrize("name", POW2)
@pytest.mark.parametrize("block", ["32", "full"])
def test_hadamard_full_size_sampled(torch_dev, kq, orc, name, block):
    torch = torch_dev
    w = synth.workload(name)
    n = 32 if block == "32" else w.d
    case("hadamard %s n=%d" % (name, n))
    A = dev_bf16(torch, w.A)
    y = torch.empty((w.m, w.d), dtype=torch.float32, device="cuda")
    codes, scales = kq.hadamard_quantize_mxfp4(A, n, y_debug=y)
    c2, s2 = kq.hadamard_quantize_mxfp4(A, n)
    torch.cuda.synchronize()
    assert torch.equal(codes, c2) and torch.equal(scales, s2)
    nrows = 64 if n <= 4096 else 12
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, w.m - 1], rng.choice(w.m, nrows, replace=False)]))
    idx = torch.from_numpy(rows).to("cuda")
    g = lambda t: t.index_select(0, idx).cpu().numpy()
    Ar = w.A[rows]
    _, _, yr = orc.hadamard_quantize(Ar, n, want_codes=False)
    rep = parity.fused_report(orc, Ar, None, g(codes), g(scales), g(y), y_ref=yr)
    print("[parity] hadamard %s n=%d rows=%d: %s" % (name, n, len(rows), rep), flush=True)
