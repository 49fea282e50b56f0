"""GPU parity of the W4A4 layer with its low-rank branch (Sec. 3.4 Eq. 11, App. D):
the fused quantizer's bf16 activation output, the projection Z = X16 Q(R)^T, the
GEMM with the low-rank epilogue, and the whole layer on the FLUX 18432x3072x3072
config against the oracle (oracle/lowrank.py) on sampled rows.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import lowrank

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


@pytest.mark.parametrize("m,d", [(70, 96), (256, 3072)])
def test_y16_is_rounded_y(torch_dev, kq, m, d):
    torch = torch_dev
    case("y16 %dx%d" % (m, d))
    A = synth.random_bf16_matrix(m, d, seed=m + d, scale=4.0)
    fac = torch.from_numpy(synth.lu_perturbed_factors(d // 32, 3)).cuda()
    Ad = dev_bf16(torch, A)
    y = torch.empty((m, d), dtype=torch.float32, device="cuda")
    c1, s1 = kq.transform_quantize_mxfp4(Ad, fac, y_debug=y)
    c2, s2, y16 = kq.transform_quantize_mxfp4_y16(Ad, fac)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    assert torch.equal(y16.view(torch.int16), y.to(torch.bfloat16).view(torch.int16))


def quantize_host(orc, X):
    codes, scales = orc.quantize_f64(np.asarray(X, dtype=np.float64))
    return codes, scales


@pytest.mark.parametrize("m,d,r", [(100, 96, 32), (300, 3072, 128), (64, 512, 160)])
def test_lowrank_project(torch_dev, kq, orc, m, d, r):
    torch = torch_dev
    case("project %dx%d r=%d" % (m, d, r))
    X = synth.random_bf16_matrix(m, d, seed=d + r)
    R = np.random.default_rng(r).standard_normal((r, d)) / np.sqrt(d)
    cr, sr = quantize_host(orc, R)
    Z = kq.lowrank_project(dev_bf16(torch, X), torch.from_numpy(cr).cuda(), torch.from_numpy(sr).cuda())
    torch.cuda.synchronize()
    Xf = synth.bf16_bits_to_f32(X).astype(np.float64)
    Rq = orc.dequantize(cr, sr, d)
    ref = Xf @ Rq.T
    bound = 2.0 ** -22 * d * (np.abs(Xf) @ np.abs(Rq).T) + 1e-30
    assert (np.abs(Z.cpu().numpy() - ref) <= bound).all()


@pytest.mark.parametrize("rows,k,seed", [(1, 32, 1), (160, 3072, 2), (37, 96, 3)])
def test_dequantize_bf16_is_exact(torch_dev, kq, orc, rows, k, seed):
    """Every MXFP4 value has at most two significant bits: its bf16 is the oracle's
    fp64 value exactly, down to bf16 subnormals (scale bytes 1 .. 250)."""
    torch = torch_dev
    case("dequantize bf16 %dx%d" % (rows, k))
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    sc = rng.integers(1, 251, (rows, k // 32), dtype=np.uint8)
    out = kq.dequantize_mxfp4_bf16(torch.from_numpy(c).cuda(), torch.from_numpy(sc).cuda())
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, orc.dequantize(c, sc, k))


def test_dequantize_bf16_every_code_and_scale(torch_dev, kq, orc):
    """All 16 E2M1 codes under every finite E8M0 scale byte 0 .. 254: exact where the
    value fits bf16 (subnormal at byte 0, largest normal at 252), +-inf past its
    largest finite value (6 * 2^126 and up); both sides of the converts' range."""
    torch = torch_dev
    case("dequantize bf16 every code x scale byte")
    row = np.array([(j << 4) | j for j in range(16)], dtype=np.uint8)
    c = np.tile(row, (255, 1))
    sc = np.arange(255, dtype=np.uint8).reshape(255, 1)
    out = kq.dequantize_mxfp4_bf16(torch.from_numpy(c).cuda(), torch.from_numpy(sc).cuda())
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = orc.dequantize(c, sc, 32)
    big = np.abs(ref) > float(torch.finfo(torch.bfloat16).max)
    assert big.sum() == 24  # codes 4 and 6 (both signs, twice each) at byte 253; 2, 3, 4, 6 at 254
    assert np.array_equal(got[~big], ref[~big])
    assert np.array_equal(got[big], np.sign(ref[big]) * np.inf)


@pytest.mark.parametrize("m,d,r", [(100, 96, 32), (300, 3072, 128), (64, 512, 160), (1, 32, 32), (79, 800, 96),
                                   (81, 1152, 256), (241, 4608, 128), (18432, 3072, 128)])
def test_lowrank_project_bf16_matches(torch_dev, kq, orc, m, d, r):
    """R decoded once to bf16, then the projection without in-kernel decoding: the same
    R values, k order and matrix instructions, so Z is bit-identical."""
    torch = torch_dev
    case("project bf16 %dx%d r=%d" % (m, d, r))
    X = synth.random_bf16_matrix(m, d, seed=d + r + 7)
    R = np.random.default_rng(r + 7).standard_normal((r, d)) / np.sqrt(d)
    cr, sr = quantize_host(orc, R)
    dcr, dsr = torch.from_numpy(cr).cuda(), torch.from_numpy(sr).cuda()
    dX = dev_bf16(torch, X)
    Z = kq.lowrank_project(dX, dcr, dsr)
    Z16 = kq.lowrank_project_bf16(dX, kq.dequantize_mxfp4_bf16(dcr, dsr))
    torch.cuda.synchronize()
    assert torch.equal(Z, Z16)


@pytest.mark.parametrize("m,d,r", [(100, 96, 32), (300, 3072, 128), (81, 1152, 256), (18432, 3072, 128)])
def test_lowrank_project_bf16_split_is_split_of_z(torch_dev, kq, orc, m, d, r):
    """The split-output projection writes bf16(Z) and bf16(Z - bf16(Z)) of the very Z the
    fp32-output projection computes, bit for bit."""
    torch = torch_dev
    case("project bf16 split %dx%d r=%d" % (m, d, r))
    X = synth.random_bf16_matrix(m, d, seed=d + r + 11)
    R = np.random.default_rng(r + 11).standard_normal((r, d)) / np.sqrt(d)
    cr, sr = quantize_host(orc, R)
    r16 = kq.dequantize_mxfp4_bf16(torch.from_numpy(cr).cuda(), torch.from_numpy(sr).cuda())
    dX = dev_bf16(torch, X)
    Z = kq.lowrank_project_bf16(dX, r16)
    Zh, Zl = kq.lowrank_project_bf16_split(dX, r16)
    torch.cuda.synchronize()
    eh = Z.to(torch.bfloat16)
    el = (Z - eh.float()).to(torch.bfloat16)
    assert torch.equal(Zh.view(torch.int16), eh.view(torch.int16))
    assert torch.equal(Zl.view(torch.int16), el.view(torch.int16))


@pytest.mark.parametrize("m,d,r,edge", [(100, 96, 32, False), (300, 3072, 128, False), (81, 1152, 256, False),
                                        (333, 160, 64, True), (18432, 3072, 128, False)])
def test_lowrank_project_mx_r_is_decoded_r(torch_dev, kq, orc, m, d, r, edge):
    """R in MXFP4, decoded by the projection's producer waves (hardware convert, the
    arithmetic decode for scale bytes outside 2..252): Z and its bf16 split bit for bit
    those of the bf16-R projection on kq_dequantize_mxfp4_bf16 of R. d = 96 and 160
    end inside a 128-k step; `edge` puts scale bytes 0, 1, 253 and 254 in R."""
    torch = torch_dev
    case("project mx R %dx%d r=%d edge=%s" % (m, d, r, edge))
    X = synth.random_bf16_matrix(m, d, seed=d + r + 31, scale=0.25 if edge else 1.0)
    R = np.random.default_rng(r + d + 31).standard_normal((r, d)) / np.sqrt(d)
    cr, sr = quantize_host(orc, R)
    if edge:
        sr = sr.copy()
        sr[0, 0], sr[1, -1], sr[r - 1, 1], sr[r // 2, 2] = 0, 1, 253, 254
    dX = dev_bf16(torch, X)
    dcr, dsr = torch.from_numpy(cr).cuda(), torch.from_numpy(sr).cuda()
    r16 = kq.dequantize_mxfp4_bf16(dcr, dsr)
    Z = kq.lowrank_project(dX, dcr, dsr)
    Zr = kq.lowrank_project_bf16(dX, r16)
    Zh, Zl = kq.lowrank_project_split(dX, dcr, dsr)
    Zhr, Zlr = kq.lowrank_project_bf16_split(dX, r16)
    torch.cuda.synchronize()
    assert torch.equal(Z.view(torch.int32), Zr.view(torch.int32))
    assert torch.equal(Zh.view(torch.int16), Zhr.view(torch.int16))
    assert torch.equal(Zl.view(torch.int16), Zlr.view(torch.int16))


def test_lowrank_project_bf16_strided_x(torch_dev, kq, orc):
    """X16 a row-strided view (ldx = d + 64) over several 80-row tiles and a ragged last
    one: the same Z, bit for bit, as the in-workgroup decode path on the same view, and the
    split-output form writes its bf16 split."""
    torch = torch_dev
    m, d, r, pad = 333, 1152, 96, 64
    case("project bf16 strided X %dx%d ldx=%d r=%d" % (m, d, d + pad, r))
    Xw = synth.random_bf16_matrix(m, d + pad, seed=21)
    R = np.random.default_rng(22).standard_normal((r, d)) / np.sqrt(d)
    cr, sr = quantize_host(orc, R)
    dcr, dsr = torch.from_numpy(cr).cuda(), torch.from_numpy(sr).cuda()
    dX = dev_bf16(torch, Xw)[:, :d]
    assert dX.stride(0) == d + pad
    Z = kq.lowrank_project(dX, dcr, dsr)
    Z16 = kq.lowrank_project_bf16(dX, kq.dequantize_mxfp4_bf16(dcr, dsr))
    Zc = kq.lowrank_project_bf16(dX.contiguous(), kq.dequantize_mxfp4_bf16(dcr, dsr))
    Zh, Zl = kq.lowrank_project_bf16_split(dX, kq.dequantize_mxfp4_bf16(dcr, dsr))
    torch.cuda.synchronize()
    assert torch.equal(Z, Z16) and torch.equal(Z16, Zc)
    eh = Z16.to(torch.bfloat16)
    assert torch.equal(Zh.view(torch.int16), eh.view(torch.int16))
    assert torch.equal(Zl.view(torch.int16), (Z16 - eh.float()).to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("m,n,k,r", [(130, 70, 96, 32), (256, 256, 512, 128), (200, 130, 256, 160)])
def test_gemm_lowrank_epilogue(torch_dev, kq, orc, m, n, k, r):
    torch = torch_dev
    case("gemm lowrank %dx%dx%d r=%d" % (m, n, k, r))
    rng = np.random.default_rng(m + n + k + r)
    ca, sa = quantize_host(orc, rng.standard_normal((m, k)))
    cw, sw = quantize_host(orc, rng.standard_normal((n, k)) / np.sqrt(k))
    cl, sl = quantize_host(orc, rng.standard_normal((n, r)) / np.sqrt(r))
    Z = (rng.standard_normal((m, r)) * 3.0).astype(np.float32)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    O = kq.mxfp4_gemm_lowrank(t(ca), t(sa), t(cw), t(sw), t(Z), t(cl), t(sl))
    O0 = kq.mxfp4_gemm(t(ca), t(sa), t(cw), t(sw))
    torch.cuda.synchronize()
    Lq = orc.dequantize(cl, sl, r)
    low = Z.astype(np.float64) @ Lq.T
    ref = orc.gemm_dequant(ca, sa, cw, sw, k) + low
    # the split of Z is exact to 2^-16 relative; fp32 sums add a few 2^-24 per term
    bound = (2.0 ** -15 + r * 2.0 ** -23) * (np.abs(Z.astype(np.float64)) @ np.abs(Lq).T) + \
        2.0 ** -20 * np.abs(ref) + 1e-30
    assert (np.abs(O.cpu().numpy() - ref) <= bound).all()
    # without the branch the epilogue kernel is the plain GEMM
    assert np.allclose(O.cpu().numpy() - low, O0.cpu().numpy(), rtol=0, atol=1e-4 * np.abs(low).max())


@pytest.fixture(scope="module")
def flux_layer(torch_dev, kq, orc):
    """Eq. 11 on the FLUX 18432x3072 activations with the 3072x3072 weights and the
    workload's factors; L, R (rank 128) are the top singular pairs of W T^{-T},
    computed offline on the host. GPU side shared by both routes: fold, residual
    W~ - L R (fp32 GEMM), MXFP4 of the residual, of L and of R, the fused transform
    + quantize with the bf16 output. Oracle: the layer on 96 sampled rows."""
    torch = torch_dev
    w = synth.workload("flux_18432x3072")
    W = synth.weights(3072, 3072, 1004)
    fac = w.factors
    r = 128
    Wt = orc.inverse_fold(W, fac)
    U, S, Vt = np.linalg.svd(Wt, full_matrices=False)
    L = (U[:, :r] * S[:r]).astype(np.float32)
    R = Vt[:r].astype(np.float32)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    facd, Ld, Rd = t(fac), t(L), t(R)
    A = dev_bf16(torch, w.A)
    Wtd = kq.inverse_fold_weights(t(W), facd)
    resid = kq.gemm_f32(Ld, Rd, alpha=-1.0, beta=1.0, C=Wtd)
    cw, sw = kq.quantize_mxfp4_f32(resid)
    cr, sr = kq.quantize_mxfp4_f32(Rd)
    cl, sl = kq.quantize_mxfp4_f32(Ld)
    ca, sa, y16 = kq.transform_quantize_mxfp4_y16(A, facd)
    cw0, sw0 = kq.quantize_mxfp4_f32(Wtd)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(13).choice(w.m, 96, replace=False))
    ref, _ = lowrank.layer(w.A[rows], W, fac, L.astype(np.float64), R.astype(np.float64), orc)
    exact = synth.bf16_bits_to_f32(w.A[rows]).astype(np.float64) @ W.astype(np.float64).T
    return dict(r=r, rows=rows, idx=torch.from_numpy(rows).cuda(), ref=ref, exact=exact, ca=ca, sa=sa, y16=y16,
                cw=cw, sw=sw, cr=cr, sr=sr, cl=cl, sl=sl, cw0=cw0, sw0=sw0)


def _report(torch, F, O, route):
    og = O.index_select(0, F["idx"]).cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(og - F["ref"]) / np.linalg.norm(F["ref"])
    print("[lowrank] %s: rel(gpu layer vs oracle) %.2e; |O - A W^T| with the rank-%d branch %.2f" % (
        route, rel, F["r"], np.linalg.norm(og - F["exact"])), flush=True)
    return rel


def test_lowrank_layer_flux(torch_dev, kq, flux_layer):
    """The check-GEMM route: projection with in-kernel decoding of R, then the
    16x16x128-instruction GEMM with the low-rank epilogue."""
    torch, F = torch_dev, flux_layer
    case("lowrank layer 18432x3072x3072 r=128, check-GEMM route")
    Z = kq.lowrank_project(F["y16"], F["cr"], F["sr"])
    O = kq.mxfp4_gemm_lowrank(F["ca"], F["sa"], F["cw"], F["sw"], Z, F["cl"], F["sl"])
    O0 = kq.mxfp4_gemm(F["ca"], F["sa"], F["cw0"], F["sw0"])
    torch.cuda.synchronize()
    rel = _report(torch, F, O, "check route")
    e_plain = np.linalg.norm(O0.index_select(0, F["idx"]).cpu().numpy().astype(np.float64) - F["exact"])
    print("[lowrank] |O - A W^T| without the branch %.2f" % e_plain, flush=True)
    assert rel <= 1e-3


def test_lowrank_layer_flux_packed_route(torch_dev, kq, flux_layer):
    """The route the layer timing measures: R decoded once to bf16, the projection on
    bf16 R, the activation scales packed, and the packed-scale GEMM with the low-rank
    epilogue (whole rounds of 256 x 256 tiles, then the last partial round as half
    tiles). Sampled rows against the oracle's layer; every element against the check
    route (the same sum in another order)."""
    torch, F = torch_dev, flux_layer
    case("lowrank layer 18432x3072x3072 r=128, packed route")
    r16 = kq.dequantize_mxfp4_bf16(F["cr"], F["sr"])
    Z = kq.lowrank_project_bf16(F["y16"], r16)
    psa, psw = kq.pack_mxfp4_scales(F["sa"]), kq.pack_mxfp4_scales(F["sw"])
    O = kq.mxfp4_gemm_packed_lowrank(F["ca"], psa, F["cw"], psw, Z, F["cl"], F["sl"])
    Zc = kq.lowrank_project(F["y16"], F["cr"], F["sr"])
    Oc = kq.mxfp4_gemm_lowrank(F["ca"], F["sa"], F["cw"], F["sw"], Zc, F["cl"], F["sl"])
    torch.cuda.synchronize()
    assert torch.equal(Z, Zc)
    rel = _report(torch, F, O, "packed route")
    assert rel <= 1e-3
    # the two GEMMs differ only in fp32 rounding of partial sums: bound each output by
    # the row's largest |term| sums (codes of A times the largest |W~| and |L| per k)
    d = (O - Oc).abs()
    scale = Oc.abs().amax(dim=1, keepdim=True) + 1.0
    worst = float((d / scale).max())
    print("[lowrank] packed vs check route: max |diff| / (row max + 1) %.3g" % worst, flush=True)
    assert worst <= 1e-4


def test_lowrank_layer_flux_split_route(torch_dev, kq, flux_layer):
    """The route with the branch's operands prepared once: the projection writes Z's bf16
    split, L is decoded to bf16 once, and the packed GEMM moves both straight into LDS.
    Bit-identical to the packed route (same Z, same instructions and order); sampled rows
    against the oracle's layer."""
    torch, F = torch_dev, flux_layer
    case("lowrank layer 18432x3072x3072 r=128, split-operand route")
    r16 = kq.dequantize_mxfp4_bf16(F["cr"], F["sr"])
    Zh, Zl = kq.lowrank_project_bf16_split(F["y16"], r16)
    psa, psw = kq.pack_mxfp4_scales(F["sa"]), kq.pack_mxfp4_scales(F["sw"])
    O = kq.mxfp4_gemm_packed_lowrank_split(F["ca"], psa, F["cw"], psw, Zh, Zl,
                                           kq.dequantize_mxfp4_bf16(F["cl"], F["sl"]))
    Z = kq.lowrank_project_bf16(F["y16"], r16)
    Op = kq.mxfp4_gemm_packed_lowrank(F["ca"], psa, F["cw"], psw, Z, F["cl"], F["sl"])
    torch.cuda.synchronize()
    assert torch.equal(O, Op)
    rel = _report(torch, F, O, "split-operand route")
    assert rel <= 1e-3
