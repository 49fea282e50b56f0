"""GPU parity of the W4A4 products on 128 x 512 output tiles: the plain MXFP4 GEMM
(kq_mxfp4_gemm_wide) against the 128 x 128 kernel (bit-identical) and the oracle's
dequantized fp64 product, and the layer with the Kronecker transform and the MXFP4
quantizer inside the product's prologue (kq_transform_quantize_mxfp4_gemm) against
the two-launch pipeline (bit-identical when every block admits the shear form) and
against the oracle's pipeline from the same seeded inputs.
"""
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


def dev_bf16(torch, A):
    return torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).cuda().view(torch.bfloat16)


def dev(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def weights_mxfp4(torch, kq, W, fac):
    """The weight side of the layer: fold W T^{-T}, then the fp32 quantizer (GPU)."""
    Wf = kq.inverse_fold_weights(dev(torch, W), dev(torch, fac))
    return kq.quantize_mxfp4_f32(Wf)


@pytest.mark.parametrize("m,n,k,seed", [(128, 512, 128, 1), (1, 1, 32, 2), (37, 70, 160, 3),
                                        (300, 1100, 416, 4), (129, 513, 96, 5), (64, 600, 4096, 6)])
def test_wide_gemm_matches_gemm_and_oracle(torch_dev, kq, orc, m, n, k, seed):
    """Seeded random MXFP4 operands (any code byte, scales around 2^0); ragged m and n,
    k not a multiple of 128 and k/32 not a multiple of 4. The wide kernel runs the
    32 x 32 x 64 instruction in ascending k, as the packed-scale GEMM does: bit-identical
    to it where that one applies (k % 256 == 0); against the 16 x 16 x 128 kernel and
    the fp64 product, fp32 accumulation accuracy."""
    torch = torch_dev
    case("wide gemm m=%d n=%d k=%d" % (m, n, k))
    rng = np.random.default_rng(seed)
    ca = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sa = rng.integers(118, 136, (m, k // 32), dtype=np.uint8)
    sw = rng.integers(118, 136, (n, k // 32), dtype=np.uint8)
    ops = [dev(torch, x) for x in (ca, sa, cw, sw)]
    O_wide = kq.mxfp4_gemm_wide(*ops)
    O_ref_kernel = kq.mxfp4_gemm(*ops)
    if k % 256 == 0:
        O_packed = kq.mxfp4_gemm_packed(ops[0], kq.pack_mxfp4_scales(ops[1]), ops[2], kq.pack_mxfp4_scales(ops[3]))
    torch.cuda.synchronize()
    if k % 256 == 0:
        assert torch.equal(O_wide, O_packed)
    ref = orc.gemm_dequant(ca, sa, cw, sw, k)
    got = O_wide.cpu().numpy().astype(np.float64)
    absdot = np.abs(orc.dequantize(ca, sa, k)) @ np.abs(orc.dequantize(cw, sw, k)).T
    assert np.all(np.abs(got - ref) <= 64 * 2.0 ** -24 * absdot + 1e-30)
    other = O_ref_kernel.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - other) <= 128 * 2.0 ** -24 * absdot + 1e-30)


def test_wide_gemm_padded_output_and_guard(torch_dev, kq):
    """ldo > n: the padding columns and the bytes after O stay untouched."""
    torch = torch_dev
    case("wide gemm ldo > n, guard")
    rng = np.random.default_rng(11)
    m, n, k, ldo = 200, 530, 256, 560
    ca = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sa = rng.integers(120, 134, (m, k // 32), dtype=np.uint8)
    sw = rng.integers(120, 134, (n, k // 32), dtype=np.uint8)
    ops = [dev(torch, x) for x in (ca, sa, cw, sw)]
    buf = torch.full((m * ldo + 1024,), 7.5, dtype=torch.float32, device="cuda")
    O = buf[: m * ldo].view(m, ldo)[:, :n]
    kq.mxfp4_gemm_wide(*ops, out=O)
    ref = kq.mxfp4_gemm_packed(ops[0], kq.pack_mxfp4_scales(ops[1]), ops[2], kq.pack_mxfp4_scales(ops[3]))
    torch.cuda.synchronize()
    assert torch.equal(O, ref)
    assert bool((buf[: m * ldo].view(m, ldo)[:, n:] == 7.5).all())
    assert bool((buf[m * ldo:] == 7.5).all())


@pytest.mark.parametrize("m,k,n,pad", [(37, 160, 70, 0), (300, 3072, 600, 8), (129, 416, 513, 0)])
def test_fused_layer_matches_pipeline_small(torch_dev, kq, orc, m, k, n, pad):
    """LU-perturbed factors (every block in shear form): the fused layer equals the
    quantizer followed by the wide GEMM bit for bit (the same product kernel), and the oracle's pipeline within fp32
    accumulation accuracy of the same dequantized operands where the codes agree."""
    torch = torch_dev
    case("fused layer m=%d k=%d n=%d pad=%d" % (m, k, n, pad))
    A_full = synth.random_bf16_matrix(m, k + pad, seed=m + k, scale=2.0)
    A_full[:, 3] = synth.to_bf16_bits(np.full(m, 250.0))
    fac = synth.lu_perturbed_factors(k // 32, seed=k + 7)
    W = synth.weights(n, k, 1004 + n)
    cw, sw = weights_mxfp4(torch, kq, W, fac)
    A = dev_bf16(torch, A_full)[:, :k]
    fac_d = dev(torch, fac)
    O_fused = kq.transform_quantize_mxfp4_gemm(A, fac_d, cw, sw)
    ca, sa = kq.transform_quantize_mxfp4(A, fac_d)
    O_pipe = kq.mxfp4_gemm_wide(ca, sa, cw, sw)
    torch.cuda.synchronize()
    assert torch.equal(O_fused, O_pipe)
    # against the oracle's pipeline on the same seeded inputs
    ca_r, sa_r, _ = orc.transform_quantize(np.ascontiguousarray(A_full[:, :k]), fac, want_y=False)
    cw_r, sw_r = orc.quantize_f64(orc.inverse_fold(W, fac))
    O_r = orc.gemm_dequant(ca_r, sa_r, cw_r, sw_r, k)
    got = O_fused.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - O_r) / np.linalg.norm(O_r)
    print("[w4a4-fused] m=%d k=%d n=%d rel vs oracle pipeline %.3g" % (m, k, n, rel), flush=True)
    assert rel <= 1e-3, rel


def test_fused_layer_nonshear_blocks_against_oracle(torch_dev, kq, orc):
    """Blocks whose G2 is a swap (no shear form): their 128-channel groups run the
    general stages. Checked against the oracle's pipeline (1e-3 relative Frobenius, the
    downstream bar) and against the GPU pipeline (same bar; codes may differ at ties)."""
    torch = torch_dev
    case("fused layer non-shear blocks")
    m, k, n = 260, 640, 300
    A_full = synth.random_bf16_matrix(m, k, seed=5, scale=3.0)
    fac = synth.lu_perturbed_factors(k // 32, seed=6)
    for blk in (1, 9, 19):
        fac[blk, 1] = np.array([[0.0, 1.0], [1.0, 0.0]], np.float32)
    W = synth.weights(n, k, 1099)
    cw, sw = weights_mxfp4(torch, kq, W, fac)
    A = dev_bf16(torch, A_full)
    fac_d = dev(torch, fac)
    O_fused = kq.transform_quantize_mxfp4_gemm(A, fac_d, cw, sw)
    ca, sa = kq.transform_quantize_mxfp4(A, fac_d)
    O_pipe = kq.mxfp4_gemm_wide(ca, sa, cw, sw)
    torch.cuda.synchronize()
    ca_r, sa_r, _ = orc.transform_quantize(A_full, fac, want_y=False)
    cw_r, sw_r = orc.quantize_f64(orc.inverse_fold(W, fac))
    O_r = orc.gemm_dequant(ca_r, sa_r, cw_r, sw_r, k)
    got = O_fused.cpu().numpy().astype(np.float64)
    pipe = O_pipe.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - O_r) / np.linalg.norm(O_r)
    rel_p = np.linalg.norm(got - pipe) / np.linalg.norm(pipe)
    print("[w4a4-fused] non-shear: rel vs oracle %.3g, vs gpu pipeline %.3g" % (rel, rel_p), flush=True)
    assert rel <= 1e-3 and rel_p <= 1e-3


def test_fused_layer_exact_factors_reduce_to_plain_quantizer(torch_dev, kq):
    """Identity factors: the fused layer is the quantize-only activation times W."""
    torch = torch_dev
    case("fused layer identity factors")
    m, k, n = 150, 384, 520
    A = dev_bf16(torch, synth.random_bf16_matrix(m, k, seed=21, scale=4.0))
    fac = dev(torch, synth.special_factors(k // 32, "identity"))
    rng = np.random.default_rng(22)
    cw = dev(torch, rng.integers(0, 256, (n, k // 2), dtype=np.uint8))
    sw = dev(torch, rng.integers(120, 134, (n, k // 32), dtype=np.uint8))
    O_fused = kq.transform_quantize_mxfp4_gemm(A, fac, cw, sw)
    ca, sa = kq.quantize_mxfp4(A)
    O_q = kq.mxfp4_gemm_wide(ca, sa, cw, sw)
    torch.cuda.synchronize()
    # quantize-only writes the sign of exact zeros from the bf16 input; the transform
    # path's y is fp32 and the sign of a zero product does not change the product
    assert torch.equal(O_fused, O_q)


def test_fused_layer_flux_config4(torch_dev, kq, orc):
    """The 18432x3072 FLUX activations and the 3072x3072 folded weights. The fused layer
    equals the two-launch pipeline (quantizer, wide GEMM) bit for bit on the whole output, so its activation
    codes are the standalone quantizer's (checked against the oracle by the quantizer's
    parity rule elsewhere). On sampled rows: the product equals the fp64 product of those
    operands dequantized, to fp32 accumulation accuracy; and rows whose activation codes
    equal the oracle's match the oracle's whole pipeline to 1e-3 relative Frobenius. A
    code that differs at a rounding tie (allowed by the rule) moves its row by one E2M1
    level times a weight row, which in an outlier channel is a few percent of the row, so
    tie rows are counted and reported, not held to the layer bar."""
    torch = torch_dev
    case("fused layer 18432x3072x3072")
    w = synth.workload("flux_18432x3072")
    W = synth.weights(3072, 3072, 1004)
    fac_d = dev(torch, w.factors)
    cw, sw = weights_mxfp4(torch, kq, W, w.factors)
    A = dev_bf16(torch, w.A)
    O_fused = kq.transform_quantize_mxfp4_gemm(A, fac_d, cw, sw)
    ca, sa = kq.transform_quantize_mxfp4(A, fac_d)
    O_pipe = kq.mxfp4_gemm_wide(ca, sa, cw, sw)
    torch.cuda.synchronize()
    assert torch.equal(O_fused, O_pipe)
    rng = np.random.default_rng(8)
    rows = np.sort(rng.choice(w.m, size=128, replace=False))
    rows[0], rows[-1] = 0, w.m - 1
    ri = torch.from_numpy(rows).cuda()
    got = O_fused[ri].cpu().numpy().astype(np.float64)
    ga, gs = ca[ri].cpu().numpy(), sa[ri].cpu().numpy()
    cw_h, sw_h = cw.cpu().numpy(), sw.cpu().numpy()
    # the product of the operands the GPU used, in fp64
    O_ops = orc.gemm_dequant(ga, gs, cw_h, sw_h, 3072)
    absdot = np.abs(orc.dequantize(ga, gs, 3072)) @ np.abs(orc.dequantize(cw_h, sw_h, 3072)).T
    assert np.all(np.abs(got - O_ops) <= 64 * 2.0 ** -24 * absdot + 1e-30)
    # the oracle's own pipeline from the seeded inputs
    ca_r, sa_r, _ = orc.transform_quantize(w.A[rows], w.factors, want_y=False)
    cw_r, sw_r = orc.quantize_f64(orc.inverse_fold(W, w.factors))
    O_r = orc.gemm_dequant(ca_r, sa_r, cw_r, sw_r, 3072)
    same = np.all(ga == ca_r, axis=1) & np.all(gs == sa_r, axis=1)
    rel_all = np.linalg.norm(got - O_r) / np.linalg.norm(O_r)
    rel = np.linalg.norm(got[same] - O_r[same]) / np.linalg.norm(O_r[same])
    w_diff = int((cw_h != cw_r).sum() + (sw_h != sw_r).sum())
    print("[w4a4-fused] flux 18432x3072x3072: rows with equal activation codes %d/%d, rel vs oracle "
          "pipeline %.3g there (%.3g over all sampled rows); weight code bytes differing from the "
          "fp64 fold %d" % (same.sum(), len(rows), rel, rel_all, w_diff), flush=True)
    assert same.sum() >= len(rows) - 4
    assert rel <= 1e-3, rel
    assert w_diff <= 1e-5 * cw_h.size


@pytest.mark.parametrize("m,k,n,pad,kind", [(6000, 512, 3000, 0, "lu"), (300, 768, 520, 16, "swap"),
                                             (5, 256, 257, 0, "identity"), (1000, 1024, 700, 8, "lu")])
def test_fused_layer_against_mx_gemm(torch_dev, kq, orc, m, k, n, pad, kind):
    """The fused layer against the quantizer followed by kq_mxfp4_gemm (the 256 x 256-tile
    kernel on these k): with every block in shear form ("lu") or exact factors
    ("identity") bit for bit (the same codes, the same instructions in the same k order);
    with swap blocks (no shear form) within 1e-3 of the oracle's pipeline. Row-strided A
    (lda = k + pad), ragged m and n, several workgroup rounds (6000 x 3000)."""
    torch = torch_dev
    case("fused layer vs mx gemm m=%d k=%d n=%d pad=%d %s" % (m, k, n, pad, kind))
    A_full = synth.random_bf16_matrix(m, k + pad, seed=m + k + n, scale=2.0)
    if kind == "identity":
        fac = synth.special_factors(k // 32, "identity")
    else:
        fac = synth.lu_perturbed_factors(k // 32, seed=k + 11)
        if kind == "swap":
            for blk in (1, 9, 19):
                fac[blk, 1] = np.array([[0.0, 1.0], [1.0, 0.0]], np.float32)
    W = synth.weights(n, k, 2004 + n)
    cw, sw = weights_mxfp4(torch, kq, W, fac if kind != "identity" else synth.special_factors(k // 32, "identity"))
    A = dev_bf16(torch, A_full)[:, :k]
    fac_d = dev(torch, fac)
    O_fused = kq.transform_quantize_mxfp4_gemm(A, fac_d, cw, sw)
    if kind == "identity":
        ca, sa = kq.quantize_mxfp4(A)
    else:
        ca, sa = kq.transform_quantize_mxfp4(A, fac_d)
    O_pipe = kq.mxfp4_gemm(ca, sa, cw, sw)
    torch.cuda.synchronize()
    if kind != "swap":
        assert torch.equal(O_fused, O_pipe)
    else:
        ca_r, sa_r, _ = orc.transform_quantize(np.ascontiguousarray(A_full[:, :k]), fac, want_y=False)
        cw_r, sw_r = orc.quantize_f64(orc.inverse_fold(W, fac))
        O_r = orc.gemm_dequant(ca_r, sa_r, cw_r, sw_r, k)
        got = O_fused.cpu().numpy().astype(np.float64)
        rel = np.linalg.norm(got - O_r) / np.linalg.norm(O_r)
        print("[w4a4-fused] swap blocks: rel vs oracle pipeline %.3g" % rel, flush=True)
        assert rel <= 1e-3, rel


def test_fused_layer_empty_and_k0(torch_dev, kq):
    torch = torch_dev
    case("fused layer empty")
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    fac = torch.zeros((2, 5, 2, 2), dtype=torch.float32, device="cuda")
    cw = torch.zeros((5, 32), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((5, 2), dtype=torch.uint8, device="cuda")
    O = kq.transform_quantize_mxfp4_gemm(A, fac, cw, sw)
    assert O.shape == (0, 5)
