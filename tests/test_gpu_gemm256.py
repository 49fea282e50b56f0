"""GPU parity of the packed-scale W4A4 GEMM (kq_mxfp4_gemm_packed, 256 x 256 tiles on
the 32 x 32 x 64 scaled FP4 instruction) and of its scale re-layout
(kq_pack_mxfp4_scales): the re-layout against its definition (byte for byte), the
product against the oracle's dequantized fp64 product (per element, to fp32 rounding
of the partial sums), against kq_mxfp4_gemm (bit-identical where every fp32 partial
sum is exact), ragged shapes, padded and unaligned outputs, k = 0, and the FLUX
18432 x 3072 x 3072 layer; the fused quantizer's packed-scale output against the
re-layout of its ordinary output.
"""
import sys

import numpy as np
import pytest

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


def dev(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def packed_reference(scales):
    """[rows][k/32] -> [k/256][rows][8], written out from the layout's definition: within a
    256-k stage the even blocks 0, 2, 4, 6 first, then the odd blocks 1, 3, 5, 7."""
    rows, kb = scales.shape
    out = np.empty((kb // 8, rows, 8), dtype=np.uint8)
    for s in range(kb // 8):
        for p in range(2):
            for j in range(4):
                out[s, :, 4 * p + j] = scales[:, 8 * s + 2 * j + p]
    return out


def operands(rng, m, n, k, lo=118, hi=136):
    ca = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sa = rng.integers(lo, hi, (m, k // 32), dtype=np.uint8)
    sw = rng.integers(lo, hi, (n, k // 32), dtype=np.uint8)
    return ca, sa, cw, sw


def run_packed(torch, kq, ca, sa, cw, sw, out=None):
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    psa = kq.pack_mxfp4_scales(dsa)
    psw = kq.pack_mxfp4_scales(dsw)
    O = kq.mxfp4_gemm_packed(dca, psa, dcw, psw, out=out)
    torch.cuda.synchronize()
    return O, (dca, dsa, dcw, dsw)


def bound(orc, ca, sa, cw, sw, k):
    absdot = np.abs(orc.dequantize(ca, sa, k)) @ np.abs(orc.dequantize(cw, sw, k)).T
    return 64 * 2.0 ** -24 * absdot + 1e-30


@pytest.mark.parametrize("rows,k,seed", [(1, 256, 1), (37, 512, 2), (300, 3072, 3), (4099, 768, 4)])
def test_pack_scales_is_the_layout(torch_dev, kq, rows, k, seed):
    torch = torch_dev
    case("pack scales rows=%d k=%d" % (rows, k))
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 256, (rows, k // 32), dtype=np.uint8)
    got = kq.pack_mxfp4_scales(dev(torch, s))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().reshape(-1), packed_reference(s).reshape(-1))


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 256, 1), (37, 70, 256, 2), (257, 513, 512, 3),
                                        (300, 1100, 768, 4), (256, 256, 2304, 5), (1000, 700, 512, 6),
                                        (5632, 3000, 512, 9), (6400, 2900, 512, 11)])
def test_packed_gemm_matches_oracle(torch_dev, kq, orc, m, n, k, seed):
    """Seeded random MXFP4 operands (any code byte, scales around 2^0); ragged m and n;
    5632 x 3000 is 264 tiles, launched in the staggered order on 256 CUs; 6400 x 2900
    is 300 tiles in the plain order, 88 workgroups taking two items, two of the half
    tiles right of the last column (nothing to store)."""
    torch = torch_dev
    case("packed gemm m=%d n=%d k=%d" % (m, n, k))
    ca, sa, cw, sw = operands(np.random.default_rng(seed), m, n, k)
    O, ops = run_packed(torch, kq, ca, sa, cw, sw)
    got = O.cpu().numpy().astype(np.float64)
    ref = orc.gemm_dequant(ca, sa, cw, sw, k)
    assert np.all(np.abs(got - ref) <= bound(orc, ca, sa, cw, sw, k))
    O_old = kq.mxfp4_gemm(*ops).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - O_old) <= 2 * bound(orc, ca, sa, cw, sw, k))


@pytest.mark.parametrize("m,n,k,seed", [(300, 600, 3072, 7), (513, 257, 1024, 8), (6400, 3072, 512, 10)])
def test_packed_gemm_exact_sums_bit_identical(torch_dev, kq, orc, m, n, k, seed):
    """Scales in 2^-1 .. 2^1: every product is a multiple of 2^-4 below 144 in magnitude,
    so for k <= 3072 every fp32 partial sum is exact and all summation orders agree:
    the packed kernel, kq_mxfp4_gemm and the fp64 oracle give the same fp32 values.
    6400 x 3072 is 300 tiles: whole rounds of full tiles plus the rest as half tiles."""
    torch = torch_dev
    case("packed gemm exact sums m=%d n=%d k=%d" % (m, n, k))
    ca, sa, cw, sw = operands(np.random.default_rng(seed), m, n, k, 126, 129)
    O, ops = run_packed(torch, kq, ca, sa, cw, sw)
    O_old = kq.mxfp4_gemm(*ops)
    torch.cuda.synchronize()
    assert torch.equal(O, O_old)
    ref = orc.gemm_dequant(ca, sa, cw, sw, k)
    assert np.array_equal(O.cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("m,n,k,seed", [(12000, 6000, 512, 41), (9000, 5000, 256, 42)])
def test_packed_gemm_multi_round_exact(torch_dev, kq, orc, m, n, k, seed):
    """Launches of several rounds of workgroups on 256 CUs: 12000 x 6000 is 1128 tiles (104
    of them as halves, the staggered order, 1232 workgroups), 9000 x 5000 is 720 tiles in
    the plain order with ragged rows and columns. Scales in 2^-1 .. 2^1 make every fp32
    partial sum exact (k <= 3072): two rows of every 256-row band (so every tile) equal the
    oracle's fp64 sums rounded to fp32, every element rounds to what the bf16-output kernel
    writes, and the MX-layout product is the same bit for bit."""
    torch = torch_dev
    case("packed gemm multi-round %dx%dx%d" % (m, n, k))
    rng = np.random.default_rng(seed)
    ca, sa, cw, sw = operands(rng, m, n, k, 126, 129)
    O, ops = run_packed(torch, kq, ca, sa, cw, sw)
    dca, dsa, dcw, dsw = ops
    psa, psw = kq.pack_mxfp4_scales(dsa), kq.pack_mxfp4_scales(dsw)
    O16 = kq.mxfp4_gemm_packed(dca, psa, dcw, psw, bf16=True)
    O_mx = kq.mxfp4_gemm(dca, dsa, dcw, dsw)
    torch.cuda.synchronize()
    assert torch.equal(O.to(torch.bfloat16), O16)
    assert torch.equal(O_mx, O)
    rows = np.unique(np.concatenate([np.minimum(np.arange(0, m, 256)[:, None] + rng.integers(0, 256, (1, 2)), m - 1)
                                     .ravel(), [m - 1]]))
    ref = orc.gemm_dequant(ca, sa, cw, sw, k, rows=rows).astype(np.float32)
    assert np.array_equal(O.cpu().numpy()[rows], ref)


@pytest.mark.parametrize("ldo,off", [(260, 0), (263, 1)])
def test_packed_gemm_padded_output_and_guard(torch_dev, kq, orc, ldo, off):
    """ldo > n (16-byte stores when O is 16-byte aligned and ldo % 4 == 0, single
    stores otherwise): the padding columns and the bytes around O stay untouched."""
    torch = torch_dev
    case("packed gemm ldo=%d offset=%d" % (ldo, off))
    m, n, k = 300, 256, 512
    ca, sa, cw, sw = operands(np.random.default_rng(9), m, n, k)
    guard = 64
    buf = torch.full((off + m * ldo + guard,), -7.5, dtype=torch.float32, device="cuda")
    out = buf[off:off + m * ldo].view(m, ldo)[:, :n]
    O, _ = run_packed(torch, kq, ca, sa, cw, sw, out=out)
    whole = buf.cpu().numpy()
    assert np.all(whole[:off] == -7.5) and np.all(whole[off + m * ldo:] == -7.5)
    mat = whole[off:off + m * ldo].reshape(m, ldo)
    assert np.all(mat[:, n:] == -7.5)
    ref = orc.gemm_dequant(ca, sa, cw, sw, k)
    assert np.all(np.abs(mat[:, :n].astype(np.float64) - ref) <= bound(orc, ca, sa, cw, sw, k))


@pytest.mark.parametrize("m,n,k,r", [(130, 70, 256, 32), (256, 256, 512, 128), (300, 520, 768, 160)])
def test_packed_gemm_lowrank_matches_oracle(torch_dev, kq, orc, m, n, k, r):
    """Eq. 11 with the low-rank term in the packed GEMM's epilogue, against the oracle's
    dequantized product plus Z deq(L)^T in fp64 (ragged m, n; r not a multiple of 64)."""
    torch = torch_dev
    case("packed gemm lowrank %dx%dx%d r=%d" % (m, n, k, r))
    rng = np.random.default_rng(m + n + k + r)
    ca, sa, cw, sw = operands(rng, m, n, k)
    cl = rng.integers(0, 256, (n, r // 2), dtype=np.uint8)
    sl = rng.integers(120, 128, (n, r // 32), dtype=np.uint8)
    Z = (rng.standard_normal((m, r)) * 3.0).astype(np.float32)
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    O = kq.mxfp4_gemm_packed_lowrank(dca, kq.pack_mxfp4_scales(dsa), dcw, kq.pack_mxfp4_scales(dsw), dev(torch, Z),
                                     dev(torch, cl), dev(torch, sl))
    torch.cuda.synchronize()
    Lq = orc.dequantize(cl, sl, r)
    absz = np.abs(Z.astype(np.float64)) @ np.abs(Lq).T
    ref = orc.gemm_dequant(ca, sa, cw, sw, k) + Z.astype(np.float64) @ Lq.T
    # the split of Z is exact to 2^-16 relative; fp32 sums add a few 2^-24 per term
    b = bound(orc, ca, sa, cw, sw, k) + (2.0 ** -15 + r * 2.0 ** -23) * absz + 2.0 ** -20 * np.abs(ref)
    assert np.all(np.abs(O.cpu().numpy().astype(np.float64) - ref) <= b)


def launch_split(torch, m, n):
    """(whole tiles, tiles split into halves, staggered order) of a packed GEMM launch:
    whole rounds of 256 x 256 tiles (one per compute unit), the last partial round as
    halves when it is at most half a round; staggered when the counts divide over the
    eight XCDs (the rule of the library's work order)."""
    tiles = ((m + 255) // 256) * ((n + 255) // 256)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    rem = tiles % ncu
    split = rem if (rem > 0 and 2 * rem <= ncu) else 0
    staggered = split > 0 and tiles > rem and tiles % 8 == 0 and rem % 8 == 0 and ncu % 8 == 0
    return tiles - split, split, staggered


@pytest.mark.parametrize("m,n,k,r", [(6400, 3072, 512, 128), (6400, 3072, 512, 96), (4096, 2560, 256, 128),
                                     (5632, 3072, 512, 128), (5632, 3000, 256, 96)])
def test_packed_gemm_lowrank_full_tiles_matches_oracle(torch_dev, kq, orc, m, n, k, r):
    """The full-tile low-rank kernel on more than one round of tiles, every element
    against the oracle's fp64 Eq. 11 (product plus Z deq(L)^T): 6400 x 3072 is 300
    tiles, i.e. a round of 256 full tiles and 44 as half tiles (plain order); 4096 x
    2560 is 160 tiles, all full; 5632 x 3072 and 5632 x 3000 are 264 tiles in the
    staggered order on 256 CUs (the latter with a partial last column tile). r = 96
    leaves a partial last 64-wide chunk of the branch."""
    torch = torch_dev
    nfull, nsplit, stag = launch_split(torch, m, n)
    case("packed gemm lowrank full tiles %dx%dx%d r=%d (%d whole, %d as halves, staggered %s)" %
         (m, n, k, r, nfull, nsplit, stag))
    assert nfull > 0
    rng = np.random.default_rng(m + n + k + r + 1)
    ca, sa, cw, sw = operands(rng, m, n, k)
    cl = rng.integers(0, 256, (n, r // 2), dtype=np.uint8)
    sl = rng.integers(120, 128, (n, r // 32), dtype=np.uint8)
    Z = (rng.standard_normal((m, r)) * 3.0).astype(np.float32)
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    O = kq.mxfp4_gemm_packed_lowrank(dca, kq.pack_mxfp4_scales(dsa), dcw, kq.pack_mxfp4_scales(dsw), dev(torch, Z),
                                     dev(torch, cl), dev(torch, sl))
    torch.cuda.synchronize()
    Lq = orc.dequantize(cl, sl, r)
    Z64 = Z.astype(np.float64)
    ref = orc.gemm_dequant(ca, sa, cw, sw, k) + Z64 @ Lq.T
    b = bound(orc, ca, sa, cw, sw, k) + (2.0 ** -15 + r * 2.0 ** -23) * (np.abs(Z64) @ np.abs(Lq).T) + \
        2.0 ** -20 * np.abs(ref)
    got = O.cpu().numpy().astype(np.float64)
    bad = np.abs(got - ref) > b
    assert not bad.any(), "%d elements outside the bound, first at %s" % (bad.sum(), np.argwhere(bad)[0])


@pytest.mark.parametrize("m,n,k,pad", [(130, 70, 256, 0), (300, 520, 768, 3), (6400, 3072, 512, 0),
                                        (5632, 3000, 256, 1), (333, 2900, 512, 0), (5, 257, 1024, 2)])
def test_mx_layout_gemm_is_packed_gemm(torch_dev, kq, orc, m, n, k, pad):
    """kq_mxfp4_gemm with k a multiple of 256 runs the 256 x 256-tile kernel on the
    MX-layout scales (each stage's eight bytes per row gathered from [rows][k / 32]):
    bit for bit the packed-scale product on the same operands, whole tiles, half tiles
    and the staggered order (6400 x 3072, 5632 x 3000), ragged rows and columns, a
    row-strided output with its padding untouched; checked against the oracle's sums too."""
    torch = torch_dev
    case("mx-layout gemm %dx%dx%d ldo=%d" % (m, n, k, n + pad))
    rng = np.random.default_rng(m + n + k + pad + 5)
    ca, sa, cw, sw = operands(rng, m, n, k)
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    ref = kq.mxfp4_gemm_packed(dca, kq.pack_mxfp4_scales(dsa), dcw, kq.pack_mxfp4_scales(dsw))
    ldo = n + pad
    buf = torch.full((m * ldo + 32,), -3.0, dtype=torch.float32, device="cuda")
    out = buf[:m * ldo].view(m, ldo)[:, :n]
    kq.mxfp4_gemm(dca, dsa, dcw, dsw, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert bool((buf[:m * ldo].view(m, ldo)[:, n:] == -3.0).all()) and bool((buf[m * ldo:] == -3.0).all())
    if m * n <= 400000:
        got = out.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - orc.gemm_dequant(ca, sa, cw, sw, k)) <= bound(orc, ca, sa, cw, sw, k))


@pytest.mark.parametrize("m,n,k,r", [(130, 70, 256, 32), (6400, 3072, 512, 128), (5632, 3000, 256, 96)])
def test_mx_layout_gemm_lowrank_is_packed(torch_dev, kq, m, n, k, r):
    """kq_mxfp4_gemm_lowrank with k a multiple of 256 runs the 256 x 256-tile kernel with
    the low-rank term, on the MX-layout scales: bit for bit the packed-scale form."""
    torch = torch_dev
    case("mx-layout gemm lowrank %dx%dx%d r=%d" % (m, n, k, r))
    rng = np.random.default_rng(m + n + k + r + 9)
    ca, sa, cw, sw = operands(rng, m, n, k)
    cl = rng.integers(0, 256, (n, r // 2), dtype=np.uint8)
    sl = rng.integers(120, 128, (n, r // 32), dtype=np.uint8)
    Z = (rng.standard_normal((m, r)) * 3.0).astype(np.float32)
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    dZ, dcl, dsl = dev(torch, Z), dev(torch, cl), dev(torch, sl)
    ref = kq.mxfp4_gemm_packed_lowrank(dca, kq.pack_mxfp4_scales(dsa), dcw, kq.pack_mxfp4_scales(dsw), dZ, dcl, dsl)
    O = kq.mxfp4_gemm_lowrank(dca, dsa, dcw, dsw, dZ, dcl, dsl)
    torch.cuda.synchronize()
    assert torch.equal(O, ref)


def test_mx_layout_gemm_scales_4_byte_aligned(torch_dev, kq, orc):
    """MX-layout scales whose base is 4-byte but not 16-byte aligned (a view 4 bytes into
    a buffer): the 256 x 256-tile kernel still takes them (its scale loads are 4 bytes
    per lane) and matches the packed-scale product bit for bit; 2-byte-aligned scales
    go to the 128 x 128 kernel, which agrees with the oracle-checked product to fp32
    accumulation accuracy."""
    torch = torch_dev
    m, n, k = 700, 600, 512
    case("mx-layout gemm misaligned scales %dx%dx%d" % (m, n, k))
    rng = np.random.default_rng(77)
    ca, sa, cw, sw = operands(rng, m, n, k)
    dca, dcw = dev(torch, ca), dev(torch, cw)
    ref = kq.mxfp4_gemm_packed(dca, kq.pack_mxfp4_scales(dev(torch, sa)), dcw, kq.pack_mxfp4_scales(dev(torch, sw)))
    for off in (4, 2):
        ba = torch.zeros(sa.size + 16, dtype=torch.uint8, device="cuda")
        bw = torch.zeros(sw.size + 16, dtype=torch.uint8, device="cuda")
        va = ba[off:off + sa.size].view(sa.shape)
        vw = bw[off:off + sw.size].view(sw.shape)
        va.copy_(torch.from_numpy(sa).cuda())
        vw.copy_(torch.from_numpy(sw).cuda())
        assert va.data_ptr() % 16 == off and vw.data_ptr() % 16 == off
        O = kq.mxfp4_gemm(dca, va, dcw, vw)
        torch.cuda.synchronize()
        if off == 4:
            assert torch.equal(O, ref)
        else:
            got, want = O.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(got - want) <= 2 * bound(orc, ca, sa, cw, sw, k))


def test_w4a4_layers_graph_replays_match_eager(torch_dev, kq):
    """The W4A4 layer's launch sequences inside a captured HIP graph: the plain layer
    (quantizer writing the packed scales, packed GEMM) and the Eq. 11 layer (quantizer
    with the bf16 activation, projection from MXFP4 R writing Z's split, GEMM with the
    low-rank term). Every replay, with eager work and synchronizations in between,
    writes the eager output bit for bit."""
    import synth
    torch = torch_dev
    m, k, n, r = 600, 512, 520, 64
    case("w4a4 layer graph replay %dx%dx%d r=%d" % (m, k, n, r))
    rng = np.random.default_rng(41)
    A = torch.from_numpy(synth.random_bf16_matrix(m, k, seed=42, scale=2.0).view(np.int16)).cuda().view(
        torch.bfloat16)
    fac = dev(torch, synth.lu_perturbed_factors(k // 32, seed=43))
    _, _, cw, sw = operands(rng, 1, n, k)
    dcw, psw = dev(torch, cw), kq.pack_mxfp4_scales(dev(torch, sw))
    cr = dev(torch, rng.integers(0, 256, (r, k // 2), dtype=np.uint8))
    sr = dev(torch, rng.integers(118, 128, (r, k // 32), dtype=np.uint8))
    L16 = kq.dequantize_mxfp4_bf16(dev(torch, rng.integers(0, 256, (n, r // 2), dtype=np.uint8)),
                                   dev(torch, rng.integers(118, 128, (n, r // 32), dtype=np.uint8)))
    ca = torch.empty((m, k // 2), dtype=torch.uint8, device="cuda")
    psa = torch.empty((m * (k // 32),), dtype=torch.uint8, device="cuda")
    y16 = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    Zh = torch.empty((m, r), dtype=torch.bfloat16, device="cuda")
    Zl = torch.empty_like(Zh)
    O1 = torch.empty((m, n), dtype=torch.float32, device="cuda")
    O2 = torch.empty_like(O1)

    def layers():
        kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=psa)
        kq.mxfp4_gemm_packed(ca, psa, dcw, psw, out=O1)
        kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=psa, y16=y16)
        kq.lowrank_project_split(y16, cr, sr, Zh=Zh, Zl=Zl)
        kq.mxfp4_gemm_packed_lowrank_split(ca, psa, dcw, psw, Zh, Zl, L16, out=O2)

    layers()
    torch.cuda.synchronize()
    ref1, ref2 = O1.clone(), O2.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layers()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layers()
    for rep in range(3):
        for t in (O1, O2, Zh, Zl, ca, psa):
            t.zero_()
        other = kq.mxfp4_gemm_packed(ca, psa, dcw, psw)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O1, ref1) and torch.equal(O2, ref2), "replay %d" % rep
        assert other.shape == ref1.shape


def test_packed_gemm_extreme_scale_bytes(torch_dev, kq, orc):
    """E8M0 scale bytes at the ends of the range the quantizer writes: on even k blocks
    A's bytes 0, 1, 2 (block scales 2^-127 .. 2^-125) against W's 180, 220, 254 (2^53 ..
    2^127), so the scale products span 2^-74 .. 2^2; on odd blocks both near 2^0. The
    packed-scale kernel and the MX-layout path agree bit for bit, and both match the fp64
    product of the dequantized operands to fp32 accumulation accuracy."""
    torch = torch_dev
    m, n, k = 300, 260, 512
    case("packed gemm extreme scale bytes %dx%dx%d" % (m, n, k))
    rng = np.random.default_rng(99)
    ca = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sa = np.empty((m, k // 32), np.uint8)
    sw = np.empty((n, k // 32), np.uint8)
    sa[:, 0::2] = rng.choice(np.array([0, 1, 2], np.uint8), size=(m, k // 64))
    sw[:, 0::2] = rng.choice(np.array([180, 220, 254], np.uint8), size=(n, k // 64))
    sa[:, 1::2] = rng.choice(np.array([126, 127, 128], np.uint8), size=(m, k // 64))
    sw[:, 1::2] = rng.choice(np.array([127, 130], np.uint8), size=(n, k // 64))
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    O = kq.mxfp4_gemm_packed(dca, kq.pack_mxfp4_scales(dsa), dcw, kq.pack_mxfp4_scales(dsw))
    O_mx = kq.mxfp4_gemm(dca, dsa, dcw, dsw)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int32), O_mx.view(torch.int32))
    got = O.cpu().numpy().astype(np.float64)
    ref = orc.gemm_dequant(ca, sa, cw, sw, k)
    assert np.isfinite(got).all()
    assert np.all(np.abs(got - ref) <= bound(orc, ca, sa, cw, sw, k))


def split_bf16(torch, Z):
    """Zh = bf16(Z), Zl = bf16(Z - Zh), both rounded to nearest even (torch's fp32 -> bf16)."""
    Zh = Z.to(torch.bfloat16)
    return Zh, (Z - Zh.float()).to(torch.bfloat16)


@pytest.mark.parametrize("m,n,k,r", [(130, 70, 256, 32), (256, 256, 512, 128), (300, 520, 768, 160),
                                     (6400, 3072, 512, 128), (5632, 3000, 256, 96), (5632, 3072, 512, 128),
                                     (100, 70, 0, 64), (333, 2900, 256, 224)])
def test_packed_gemm_lowrank_split_bit_identical(torch_dev, kq, m, n, k, r):
    """The low-rank term from operands prepared once (Z split as Zh + Zl in bf16, deq(L) in
    bf16, moved straight into LDS) against the fp32-Z form on the Z they split: the same
    instructions in the same order, so every output bit agrees. Ragged shapes, several
    32-wide chunks (r = 224: seven), whole rounds plus half tiles (6400 x 3072), the
    staggered order (5632 x 3000, 5632 x 3072), k = 0 (the term alone), and half tiles
    right of the last column (333 x 2900)."""
    torch = torch_dev
    case("packed gemm lowrank split %dx%dx%d r=%d" % (m, n, k, r))
    rng = np.random.default_rng(m + n + k + r + 7)
    ca, sa, cw, sw = operands(rng, m, n, k) if k > 0 else (np.zeros((m, 0), np.uint8), np.zeros((m, 0), np.uint8),
                                                           np.zeros((n, 0), np.uint8), np.zeros((n, 0), np.uint8))
    cl = rng.integers(0, 256, (n, r // 2), dtype=np.uint8)
    sl = rng.integers(120, 128, (n, r // 32), dtype=np.uint8)
    Z = (rng.standard_normal((m, r)) * 3.0).astype(np.float32)
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    psa, psw = kq.pack_mxfp4_scales(dsa), kq.pack_mxfp4_scales(dsw)
    dZ, dcl, dsl = dev(torch, Z), dev(torch, cl), dev(torch, sl)
    O = kq.mxfp4_gemm_packed_lowrank(dca, psa, dcw, psw, dZ, dcl, dsl)
    Zh, Zl = split_bf16(torch, dZ)
    Os = kq.mxfp4_gemm_packed_lowrank_split(dca, psa, dcw, psw, Zh, Zl, kq.dequantize_mxfp4_bf16(dcl, dsl))
    torch.cuda.synchronize()
    assert torch.equal(O, Os)


@pytest.mark.parametrize("m,n,k,r,pad", [(300, 520, 512, 96, 5), (6400, 2900, 256, 128, 3)])
def test_packed_gemm_lowrank_split_padded_output(torch_dev, kq, m, n, k, r, pad):
    """The split low-rank form writing into a row-strided output (ldo = n + pad, the row
    ends taking element stores): the same bits as into a contiguous one, and the padding
    columns and the bytes after the last row untouched."""
    torch = torch_dev
    case("packed gemm lowrank split padded %dx%dx%d r=%d ldo=%d" % (m, n, k, r, n + pad))
    rng = np.random.default_rng(m + n + k + r + pad)
    ca, sa, cw, sw = operands(rng, m, n, k)
    Zh = torch.from_numpy((rng.standard_normal((m, r)) * 3.0).astype(np.float32)).cuda().to(torch.bfloat16)
    Zl = torch.from_numpy((rng.standard_normal((m, r)) * 2.0 ** -8).astype(np.float32)).cuda().to(torch.bfloat16)
    cl = rng.integers(0, 256, (n, r // 2), dtype=np.uint8)
    sl = rng.integers(120, 128, (n, r // 32), dtype=np.uint8)
    dca, dsa, dcw, dsw = (dev(torch, x) for x in (ca, sa, cw, sw))
    psa, psw = kq.pack_mxfp4_scales(dsa), kq.pack_mxfp4_scales(dsw)
    L16 = kq.dequantize_mxfp4_bf16(dev(torch, cl), dev(torch, sl))
    ref = kq.mxfp4_gemm_packed_lowrank_split(dca, psa, dcw, psw, Zh, Zl, L16)
    ldo = n + pad
    buf = torch.full((m * ldo + 64,), -7.0, dtype=torch.float32, device="cuda")
    out = buf[:m * ldo].view(m, ldo)[:, :n]
    kq.mxfp4_gemm_packed_lowrank_split(dca, psa, dcw, psw, Zh, Zl, L16, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert bool((buf[:m * ldo].view(m, ldo)[:, n:] == -7.0).all())
    assert bool((buf[m * ldo:] == -7.0).all())


@pytest.mark.parametrize("m,n,k,pad,seed", [(1000, 700, 512, 0, 21), (300, 1100, 768, 3, 22), (257, 513, 256, 1, 23),
                                            (5632, 3072, 256, 0, 24), (5632, 3000, 256, 5, 25),
                                            (5632, 2900, 512, 0, 26), (18432, 3072, 3072, 0, 24)])
def test_packed_gemm_bf16_is_rounded_fp32(torch_dev, kq, m, n, k, pad, seed):
    """The bf16-output form equals the fp32 form rounded to nearest even, bit for bit, for
    aligned (whole 16-byte row pieces) and odd-stride or partial-tile (2-byte element
    stores) outputs; padding stays untouched."""
    torch = torch_dev
    case("packed gemm bf16 m=%d n=%d k=%d ldo=%d" % (m, n, k, n + pad))
    ca, sa, cw, sw = operands(np.random.default_rng(seed), m, n, k)
    O32, (dca, dsa, dcw, dsw) = run_packed(torch, kq, ca, sa, cw, sw)
    psa, psw = kq.pack_mxfp4_scales(dsa), kq.pack_mxfp4_scales(dsw)
    ldo = n + pad
    buf = torch.full((m * ldo + 16,), -5.0, dtype=torch.bfloat16, device="cuda")
    out = buf[:m * ldo].view(m, ldo)[:, :n]
    kq.mxfp4_gemm_packed(dca, psa, dcw, psw, out=out, bf16=True)
    torch.cuda.synchronize()
    assert torch.equal(out, O32.to(torch.bfloat16))
    whole = buf.float().cpu().numpy()
    assert np.all(whole[m * ldo:] == -5.0)
    assert np.all(whole[:m * ldo].reshape(m, ldo)[:, n:] == -5.0)


def test_packed_gemm_k0_and_empty(torch_dev, kq):
    torch = torch_dev
    case("packed gemm k=0 and empty")
    z = torch.zeros((0,), dtype=torch.uint8, device="cuda")
    ca = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    cw = torch.zeros((7, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda")
    kq.mxfp4_gemm_packed(ca, z, cw, z, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    e = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    O = kq.mxfp4_gemm_packed(e, torch.zeros((0,), dtype=torch.uint8, device="cuda"), e,
                             torch.zeros((0,), dtype=torch.uint8, device="cuda"))
    assert O.shape == (0, 0)


def test_packed_gemm_flux_layer(torch_dev, kq, orc):
    """FLUX 18432 x 3072 activations against 3072 x 3072 weights, the launch the bench
    times: every element against kq_mxfp4_gemm (fp32 rounding of different partial
    sums), sampled rows against the oracle's fp64 product."""
    torch = torch_dev
    m, n, k = 18432, 3072, 3072
    case("packed gemm flux %dx%dx%d" % (m, n, k))
    ca, sa, cw, sw = operands(np.random.default_rng(12), m, n, k)
    O, ops = run_packed(torch, kq, ca, sa, cw, sw)
    O_old = kq.mxfp4_gemm(*ops)
    torch.cuda.synchronize()
    got = O.cpu().numpy().astype(np.float64)
    old = O_old.cpu().numpy().astype(np.float64)
    # every element: both kernels are within 64 ulp-steps of the exact sum, and
    # sum_k |a_ik| max_j |w_jk| bounds every sum of |products| in row i
    wmax = np.abs(orc.dequantize(cw, sw, k)).max(axis=0)
    rowbound = np.abs(orc.dequantize(ca, sa, k)) @ wmax
    diff = np.abs(got - old)
    assert np.all(diff <= 2 * 64 * 2.0 ** -24 * rowbound[:, None] + 1e-30)
    rows = np.random.default_rng(13).choice(m, 48, replace=False)
    ref = orc.gemm_dequant(ca, sa, cw, sw, k, rows=rows)
    assert np.all(np.abs(got[rows] - ref) <= bound(orc, ca[rows], sa[rows], cw, sw, k))
    print("[gemm256] flux: max |packed - gemm| %.3g (max allowed %.3g), sampled rows vs oracle max rel %.3g" % (
        diff.max(), (2 * 64 * 2.0 ** -24 * rowbound).max(),
        np.max(np.abs(got[rows] - ref) / (np.abs(ref) + 1e-30))), flush=True)


@pytest.mark.parametrize("m,d,seed,swap", [(37, 256, 31, ()), (300, 768, 32, ()), (1000, 3072, 33, ()),
                                            (5, 1024, 34, ()), (300, 768, 35, (3, 17)), (1000, 3072, 36, (40,))])
def test_quantizer_packed_scales_equal_pack_of_scales(torch_dev, kq, m, d, seed, swap):
    """kq_transform_quantize_mxfp4_packed writes the quantizer's codes and, byte for byte,
    pack_mxfp4_scales of its scales (d = 768 leaves the last 512-channel segment half
    empty, m = 5 and 37 ragged row groups; `swap` lists blocks whose G2 is a swap, which has
    no shear form, so their segments run the general 2x2 stages); with y16, also the y16
    entry point's bf16 y. Bytes after the packed array stay untouched."""
    import synth
    torch = torch_dev
    case("quantizer packed scales m=%d d=%d swap=%s" % (m, d, swap))
    A = torch.from_numpy(synth.random_bf16_matrix(m, d, seed=seed, scale=3.0).view(np.int16)).cuda().view(
        torch.bfloat16)
    fac_h = synth.lu_perturbed_factors(d // 32, seed=seed + 1)
    for blk in swap:
        fac_h[blk, 1] = np.array([[0.0, 1.0], [1.0, 0.0]], np.float32)
    fac = dev(torch, fac_h)
    ca, sa = kq.transform_quantize_mxfp4(A, fac)
    ca16, sa16, y16 = kq.transform_quantize_mxfp4_y16(A, fac)
    guard = torch.full((m * (d // 32) + 64,), 0xEE, dtype=torch.uint8, device="cuda")
    pk = guard[:m * (d // 32)]
    cp, _, none = kq.transform_quantize_mxfp4_packed(A, fac, packed_scales=pk)
    cq, pq, yq = kq.transform_quantize_mxfp4_packed(A, fac, want_y16=True)
    ref = kq.pack_mxfp4_scales(sa)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(cp, ca) and torch.equal(pk, ref.reshape(-1))
    assert torch.equal(cq, ca16) and torch.equal(pq.reshape(-1), kq.pack_mxfp4_scales(sa16).reshape(-1))
    assert torch.equal(yq, y16)
    assert bool((guard[m * (d // 32):] == 0xEE).all())


def test_quantizer_packed_scales_flux_layer(torch_dev, kq):
    """The FLUX 18432 x 3072 input: the packed-scale quantizer feeds the packed GEMM with
    the same result as quantizer + re-layout + GEMM, bit for bit."""
    import synth
    torch = torch_dev
    case("quantizer packed scales flux 18432x3072 + gemm")
    w = synth.workload("flux_18432x3072")
    A = torch.from_numpy(w.A.view(np.int16)).cuda().view(torch.bfloat16)
    fac = dev(torch, w.factors)
    rng = np.random.default_rng(41)
    cw = dev(torch, rng.integers(0, 256, (512, 3072 // 2), dtype=np.uint8))
    sw = dev(torch, rng.integers(118, 130, (512, 3072 // 32), dtype=np.uint8))
    psw = kq.pack_mxfp4_scales(sw)
    ca, sa = kq.transform_quantize_mxfp4(A, fac)
    O_ref = kq.mxfp4_gemm_packed(ca, kq.pack_mxfp4_scales(sa), cw, psw)
    cp, pp, _ = kq.transform_quantize_mxfp4_packed(A, fac)
    O = kq.mxfp4_gemm_packed(cp, pp, cw, psw)
    torch.cuda.synchronize()
    assert torch.equal(cp, ca)
    assert torch.equal(O, O_ref)
