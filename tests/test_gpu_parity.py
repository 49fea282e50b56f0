"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Inputs come from the seeded generator (synth); the oracle never sees anything
the GPU produced except where the rule says so (rule 2 of tests/parity.py
quantizes the GPU's own fp32 y with the oracle). Full-size workloads run in
the launch configuration the bench uses; the largest one is checked on
sampled rows.
"""
import sys

import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu

FULL = ["tiny_64x256", "pixart_attn_4096x1152", "pixart_ffn_8192x4608", "flux_18432x3072"]
SAMPLED = ["flux_18432x12288"]
SAMPLE_ROWS = 1536


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
    kq.lib()  # fails loudly when libkq.so is missing
    return kq


_cache = {}


def workload(name):
    if name not in _cache:
        _cache.clear()  # keep host memory bounded: one full workload at a time
        _cache[name] = synth.workload(name)
    return _cache[name]


def dev_bf16(torch, A):
    return torch.from_numpy(A.view(np.int16)).to("cuda").view(torch.bfloat16)


def sample_rows(m, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(m, size=min(n, m), replace=False))
    rows[0], rows[-1] = 0, m - 1  # include the first and the ragged last tile
    return np.unique(rows)


def gather(torch, t, rows):
    return t.index_select(0, torch.from_numpy(rows).to(t.device)).cpu().numpy()


# ---------------------------------------------------------------------------
# bit-exact paths
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", FULL + SAMPLED)
def test_quantize_only_bit_exact(torch_dev, kq, orc, name):
    torch = torch_dev
    case("quantize_only " + name)
    w = workload(name)
    A = dev_bf16(torch, w.A)
    codes, scales = kq.quantize_mxfp4(A)
    torch.cuda.synchronize()
    rows = np.arange(w.m) if name in FULL else sample_rows(w.m, SAMPLE_ROWS)
    c_ref, s_ref = orc.quantize_bf16(w.A[rows])
    assert np.array_equal(gather(torch, scales, rows), s_ref)
    assert np.array_equal(gather(torch, codes, rows), c_ref)


@pytest.mark.parametrize("name", FULL + SAMPLED)
def test_smoothquant_bit_exact(torch_dev, kq, orc, name):
    torch = torch_dev
    case("smoothquant " + name)
    w = workload(name)
    A = dev_bf16(torch, w.A)
    inv = torch.from_numpy(w.inv_scale).cuda()
    codes, scales = kq.smoothquant_quantize_mxfp4(A, inv)
    torch.cuda.synchronize()
    rows = np.arange(w.m) if name in FULL else sample_rows(w.m, SAMPLE_ROWS)
    c_ref, s_ref = orc.smoothquant_quantize(w.A[rows], w.inv_scale)
    assert np.array_equal(gather(torch, scales, rows), s_ref)
    assert np.array_equal(gather(torch, codes, rows), c_ref)


# ---------------------------------------------------------------------------
# fused Kronecker transform + quantize
# ---------------------------------------------------------------------------

@pytest.fixture(params=["default", "butterfly", "mfma", "mfma_lds"])
def form(request):
    """Transform form of the fused calls (kq_transform_quantize_mxfp4_form); "default"
    calls kq_transform_quantize_mxfp4 itself."""
    return request.param


def fused(kq, A, fac, form, **kw):
    return kq.transform_quantize_mxfp4(A, fac, form=None if form == "default" else form, **kw)


@pytest.mark.parametrize("name", FULL + SAMPLED)
def test_fused_against_oracle(torch_dev, kq, orc, name, form):
    torch = torch_dev
    case("fused %s form=%s" % (name, form))
    w = workload(name)
    A = dev_bf16(torch, w.A)
    fac = torch.from_numpy(w.factors).cuda()
    y = torch.empty((w.m, w.d), dtype=torch.float32, device="cuda")
    codes, scales = fused(kq, A, fac, form, y_debug=y)
    codes_fast, scales_fast = fused(kq, A, fac, form)
    torch.cuda.synchronize()
    # rule 4: fast mode writes the same bytes as check mode
    assert torch.equal(codes, codes_fast) and torch.equal(scales, scales_fast)
    rows = np.arange(w.m) if name in FULL else sample_rows(w.m, SAMPLE_ROWS)
    rep = parity.fused_report(orc, w.A[rows], w.factors, gather(torch, codes, rows),
                              gather(torch, scales, rows), gather(torch, y, rows))
    print("[parity] %s %s %s" % (name, form, rep), flush=True)


@pytest.mark.parametrize("kind", ["identity", "swap", "signflip", "pow2", "mixed"])
def test_fused_exact_factors_reduce_to_quantizer(torch_dev, kq, orc, kind, form):
    torch = torch_dev
    case("fused exact factors %s form=%s" % (kind, form))
    w = workload("pixart_attn_4096x1152")
    f = synth.special_factors(w.d // 32, kind)
    A = dev_bf16(torch, w.A)
    codes, scales = fused(kq, A, torch.from_numpy(f).cuda(), form)
    torch.cuda.synchronize()
    c_ref, s_ref, _ = orc.transform_quantize(w.A, f, want_y=False)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    parity.assert_codes_equal_mod_signed_zero(codes.cpu().numpy(), c_ref, kind)
    if kind == "identity":
        q_codes, q_scales = kq.quantize_mxfp4(A)
        assert torch.equal(q_scales, scales)
        parity.assert_codes_equal_mod_signed_zero(q_codes.cpu().numpy(), codes.cpu().numpy())


def test_fused_segments_with_a_nonshear_block(torch_dev, kq, orc, form):
    """LU-perturbed factors everywhere except a few blocks whose G2 is a swap (zero
    diagonal, so no shear form): every block sharing a 16-block segment with one of
    them runs the general 2x2 stages. Ragged rows and a partial last segment."""
    torch = torch_dev
    case("fused non-shear blocks form=" + form)
    m, d = 4133, 1152
    A_full = synth.random_bf16_matrix(m, d, seed=91, scale=3.0)
    fac = synth.lu_perturbed_factors(d // 32, seed=92)
    for blk in (5, 21, 35):  # segments 0, 1 and the 4-block tail segment 2
        fac[blk, 1] = np.array([[0.0, 1.0], [1.0, 0.0]], np.float32)
    y = torch.empty((m, d), dtype=torch.float32, device="cuda")
    codes, scales = fused(kq, dev_bf16(torch, A_full), torch.from_numpy(fac).cuda(), form, y_debug=y)
    codes_fast, scales_fast = fused(kq, dev_bf16(torch, A_full), torch.from_numpy(fac).cuda(), form)
    assert torch.equal(codes, codes_fast) and torch.equal(scales, scales_fast)
    rep = parity.fused_report(orc, A_full, fac, codes.cpu().numpy(), scales.cpu().numpy(), y.cpu().numpy())
    print("[parity] non-shear blocks %s %s" % (form, rep), flush=True)


def test_fused_hadamard_worked_example(torch_dev, kq, orc, form):
    torch = torch_dev
    case("fused hadamard worked example form=" + form)
    A = np.zeros((4, 64), np.uint16)
    A[:, 3] = synth.to_bf16_bits(np.array([80.0]))[0]
    A[1, 32 + 7] = synth.to_bf16_bits(np.array([-3.0]))[0]
    codes, scales = fused(kq, dev_bf16(torch, A), torch.from_numpy(synth.hadamard_factors(2)).cuda(), form)
    n = parity.unpack(codes.cpu().numpy())
    assert scales.cpu().numpy()[0, 0] == 128
    for c in range(32):
        assert n[0, c] == 7 | (8 if bin(3 & c).count("1") % 2 else 0)
    c_ref, s_ref, _ = orc.transform_quantize(A, synth.hadamard_factors(2), want_y=False)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    parity.assert_codes_equal_mod_signed_zero(codes.cpu().numpy(), c_ref)


# ---------------------------------------------------------------------------
# exhaustive quantizer checks
# ---------------------------------------------------------------------------

def all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    return bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def test_every_bf16_alone_and_in_context(torch_dev, kq, orc):
    torch = torch_dev
    case("exhaustive bf16 quantize")
    b = all_finite_bf16()
    n = b.size
    rng = np.random.default_rng(4)
    blocks = []
    # alone in a block (position varies)
    alone = np.zeros((n, 32), np.uint16)
    alone[np.arange(n), np.arange(n) % 32] = b
    blocks.append(alone)
    # every value beside a block maximum from every binade (scale contexts)
    ctx = np.zeros((n, 32), np.uint16)
    ctx[:, :31] = b[rng.integers(0, n, (n, 31))]
    ctx[:, 31] = b
    blocks.append(ctx)
    # 32 consecutive patterns per block
    m32 = (n // 32) * 32
    blocks.append(b[:m32].reshape(-1, 32))
    A = np.concatenate(blocks, axis=0)
    pad = (-A.shape[0]) % 8
    A = np.concatenate([A, np.zeros((pad, 32), np.uint16)], axis=0)
    A = np.ascontiguousarray(A.reshape(-1, 256))
    codes, scales = kq.quantize_mxfp4(dev_bf16(torch, A))
    c_ref, s_ref = orc.quantize_bf16(A)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


def boundary_f32_blocks(rng, nblocks):
    """fp32 blocks whose elements sit on and next to every E2M1 rounding boundary."""
    bounds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 0.5, 1.0, 3.0, 4.0],
                      dtype=np.float32)
    X = np.zeros((nblocks, 32), np.float32)
    e = rng.integers(-126, 125, nblocks)
    for i in range(nblocks):
        sc = np.float32(2.0) ** np.float32(e[i]) if e[i] > -126 else np.float32(2.0 ** -126)
        v = bounds[rng.integers(0, bounds.size, 31)]
        k = rng.integers(-3, 4, 31)
        vals = np.array([np.float32(x) for x in v]) * sc
        for j in range(31):
            for _ in range(abs(k[j])):
                vals[j] = np.nextafter(vals[j], np.float32(np.inf if k[j] > 0 else 0))
        sign = np.where(rng.integers(0, 2, 31) == 1, -1, 1).astype(np.float32)
        X[i, :31] = vals * sign
        X[i, 31] = np.float32(rng.choice([4.0, 6.0, 7.5])) * sc
    return X


def test_f32_quantizer_at_rounding_boundaries(torch_dev, kq, orc):
    torch = torch_dev
    case("fp32 quantize boundaries")
    rng = np.random.default_rng(6)
    X = boundary_f32_blocks(rng, 4096).reshape(512, 256)
    codes, scales = kq.quantize_mxfp4_f32(torch.from_numpy(X).cuda())
    c_ref, s_ref = orc.quantize_f32(X)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


# ---------------------------------------------------------------------------
# shapes, strides, streams, guard bytes, determinism
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,d", [(4096, 12288), (4099, 4096), (8192, 4608), (2000, 3072)])
def test_mfma_lds_form_tile_counts(torch_dev, kq, orc, m, d):
    """The LDS-staged MFMA form sizes its workgroups' runs of 16-token tiles from the launch
    (8 tiles at 4096 x 12288, 6 at 8192 x 4608, 2 at 4099 x 4096 with a last run of one
    ragged tile, 1 at 2000 x 3072): one row of every tile (so every tile of every run) and
    the last row against the oracle, and the fast mode writes the same bytes."""
    torch = torch_dev
    case("mfma_lds tile counts m=%d d=%d" % (m, d))
    A_host = synth.random_bf16_matrix(m, d, seed=m + d, scale=3.0)
    A_host[:, 7] = synth.to_bf16_bits(np.full(m, 250.0))
    fac = synth.lu_perturbed_factors(d // 32, seed=d + 3)
    A = dev_bf16(torch, A_host)
    y = torch.empty((m, d), dtype=torch.float32, device="cuda")
    codes, scales = kq.transform_quantize_mxfp4(A, torch.from_numpy(fac).cuda(), y_debug=y, form="mfma_lds")
    codes_fast, scales_fast = kq.transform_quantize_mxfp4(A, torch.from_numpy(fac).cuda(), form="mfma_lds")
    torch.cuda.synchronize()
    assert torch.equal(codes, codes_fast) and torch.equal(scales, scales_fast)
    rng = np.random.default_rng(m)
    rows = np.unique(np.concatenate([np.minimum(np.arange(0, m, 16) + rng.integers(0, 16, (m + 15) // 16), m - 1),
                                     [m - 1]]))
    rep = parity.fused_report(orc, A_host[rows], fac, gather(torch, codes, rows), gather(torch, scales, rows),
                              gather(torch, y, rows))
    print("[parity] mfma_lds m=%d d=%d %s" % (m, d, rep), flush=True)


@pytest.mark.parametrize("m,d,pad", [(1, 32, 0), (3, 96, 8), (37, 160, 0), (4133, 1152, 64),
                                     (517, 4608, 0), (70, 512, 24), (1, 12288, 0)])
def test_ragged_shapes_and_padded_rows(torch_dev, kq, orc, m, d, pad, form):
    torch = torch_dev
    case("ragged m=%d d=%d pad=%d form=%s" % (m, d, pad, form))
    A_full = synth.random_bf16_matrix(m, d + pad, seed=m * 7 + d, scale=3.0)
    A_full[:, min(5, d - 1)] = synth.to_bf16_bits(np.full(m, 300.0))
    fac = synth.lu_perturbed_factors(d // 32, seed=d + 1)
    inv = synth.smoothquant_inv_scale(A_full, d)
    A = dev_bf16(torch, A_full)[:, :d]
    assert A.stride(0) == d + pad
    codes, scales = kq.quantize_mxfp4(A)
    c_ref, s_ref = orc.quantize_bf16(A_full, d=d)
    assert np.array_equal(codes.cpu().numpy(), c_ref) and np.array_equal(scales.cpu().numpy(), s_ref)
    codes, scales = kq.smoothquant_quantize_mxfp4(A, torch.from_numpy(inv).cuda())
    c_ref, s_ref = orc.smoothquant_quantize(A_full, inv, d=d)
    assert np.array_equal(codes.cpu().numpy(), c_ref) and np.array_equal(scales.cpu().numpy(), s_ref)
    y = torch.empty((m, d), dtype=torch.float32, device="cuda")
    codes, scales = fused(kq, A, torch.from_numpy(fac).cuda(), form, y_debug=y)
    parity.fused_report(orc, np.ascontiguousarray(A_full[:, :d]), fac, codes.cpu().numpy(),
                        scales.cpu().numpy(), y.cpu().numpy())


def test_guard_bytes_determinism_and_side_stream(torch_dev, kq, form):
    torch = torch_dev
    case("guard bytes / determinism / stream form=" + form)
    w = workload("pixart_attn_4096x1152")
    m, d = w.m, w.d
    A = dev_bf16(torch, w.A)
    fac = torch.from_numpy(w.factors).cuda()
    G = 4096
    cbuf = torch.full((m * d // 2 + G,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((m * d // 32 + G,), 0x5A, dtype=torch.uint8, device="cuda")
    codes = cbuf[: m * d // 2].view(m, d // 2)
    scales = sbuf[: m * d // 32].view(m, d // 32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fused(kq, A, fac, form, codes=codes, scales=scales, stream=s)
    s.synchronize()
    assert bool((cbuf[m * d // 2:] == 0xA5).all()) and bool((sbuf[m * d // 32:] == 0x5A).all())
    c2, s2 = fused(kq, A, fac, form)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes) and torch.equal(s2, scales)


def test_fused_tiny_and_mixed_magnitudes(torch_dev, kq, orc, form):
    """Blocks of bf16 subnormals, of values near the bottom of the normal range and of
    mixed magnitudes spanning 60 binades."""
    torch = torch_dev
    case("fused tiny magnitudes form=" + form)
    rng = np.random.default_rng(12)
    m, d = 96, 256
    X = rng.standard_normal((m, d))
    X[:32] *= 2.0 ** -130      # subnormal bf16
    X[32:64] *= 2.0 ** -120    # small normals
    X[64:] *= 2.0 ** rng.integers(-30, 30, (32, d))
    A = synth.to_bf16_bits(X)
    fac = synth.lu_perturbed_factors(d // 32, 77)
    y = torch.empty((m, d), dtype=torch.float32, device="cuda")
    codes, scales = fused(kq, dev_bf16(torch, A), torch.from_numpy(fac).cuda(), form, y_debug=y)
    rep = parity.fused_report(orc, A, fac, codes.cpu().numpy(), scales.cpu().numpy(), y.cpu().numpy())
    print("[parity] tiny %s %s" % (form, rep), flush=True)


def shear_growth(fac):
    """Per block and factor, max(|G01 / G11|, |G10 / G00|): the ratios of the fused
    entry point's fp32 shear stages, which set its range condition."""
    g = fac.astype(np.float64)
    return np.maximum(np.abs(g[:, :, 0, 1] / g[:, :, 1, 1]), np.abs(g[:, :, 1, 0] / g[:, :, 0, 0]))


@pytest.mark.parametrize("kind", ["hadamard", "lu"])
def test_fused_top_of_range(torch_dev, kq, orc, kind, form):
    """Blocks near the top of the exponent range, inside the fused entry point's
    stated range condition (max|a| prod_k (1 + r_k) < 2^128, r_k the shear ratios):
    dense blocks scaled to just inside it, and blocks of one nonzero element, whose
    stages grow it only by prod_k max(1, r_k), up to the largest finite bf16 (for
    Hadamard factors that is y = 2^125.5, scale byte 250). Checked by the same rules
    as every fused run."""
    torch = torch_dev
    case("fused top of range %s form=%s" % (kind, form))
    rng = np.random.default_rng(31 if kind == "hadamard" else 32)
    m, d = 64, 512
    nblk = d // 32
    fac = synth.hadamard_factors(nblk) if kind == "hadamard" else synth.lu_perturbed_factors(nblk, 33)
    r = shear_growth(fac)
    dense = np.log2(np.prod(1.0 + r, axis=1))           # [nblk]
    spike = np.log2(np.prod(np.maximum(1.0, r), axis=1))
    X = np.zeros((m, d))
    z = np.clip(rng.standard_normal((32, d)), -4.0, 4.0)
    e = np.floor(126.5 - 2.0 - dense)[None, :] - rng.integers(0, 4, (32, nblk))
    X[:32] = z * np.repeat(2.0 ** e, 32, axis=1)
    for i in range(32, m):
        for b in range(nblk):
            lim = min(127.99, 127.9 - spike[b])
            X[i, 32 * b + (i * 7 + b) % 32] = (-1) ** (i + b) * 2.0 ** (lim - rng.uniform(0, 2) * (i % 2))
    A = synth.to_bf16_bits(X)
    y = torch.empty((m, d), dtype=torch.float32, device="cuda")
    codes, scales = fused(kq, dev_bf16(torch, A), torch.from_numpy(fac).cuda(), form, y_debug=y)
    torch.cuda.synchronize()
    rep = parity.fused_report(orc, A, fac, codes.cpu().numpy(), scales.cpu().numpy(), y.cpu().numpy())
    top_byte = int(scales.cpu().numpy().max())
    print("[parity] top of range %s %s: largest scale byte %d, %s" % (kind, form, top_byte, rep), flush=True)
    assert top_byte >= (250 if kind == "hadamard" else 245)


def test_smoothquant_top_of_range(torch_dev, kq, orc):
    """SmoothQuant with inputs up to the largest finite bf16 and per-channel factors in
    [1/2, 1]: every product is finite, and the scale bytes reach 252, the largest any
    finite fp32 block maximum gives (e = 127 - 2); bit-exact."""
    torch = torch_dev
    case("smoothquant top of range")
    rng = np.random.default_rng(34)
    m, d = 256, 256
    X = rng.uniform(-1.0, 1.0, (m, d)) * 2.0 ** rng.integers(100, 128, (m, 1))
    X = np.clip(X, -3.3e38, 3.3e38)
    A = synth.to_bf16_bits(X)
    A[0, :] = 0x7F7F  # the largest finite bf16, 2^127 (2 - 2^-7)
    A[1, 1::2] = 0xFF7F
    inv = rng.uniform(0.5, 1.0, d).astype(np.float32)
    inv[:8] = 1.0
    codes, scales = kq.smoothquant_quantize_mxfp4(dev_bf16(torch, A), torch.from_numpy(inv).cuda())
    torch.cuda.synchronize()
    c_ref, s_ref = orc.smoothquant_quantize(A, inv)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert int(s_ref.max()) == 252


@pytest.mark.parametrize("kind", ["fused", "smoothquant", "quantize"])
def test_hip_graph_replays_match_eager(torch_dev, kq, kind):
    """The kernels inside a captured HIP graph (as bench.py replays them): every
    replay, with eager work and synchronizations in between, writes the eager bytes."""
    torch = torch_dev
    case("hip graph replay " + kind)
    w = workload("pixart_attn_4096x1152")
    A = dev_bf16(torch, w.A)
    fac = torch.from_numpy(w.factors).cuda()
    inv = torch.from_numpy(w.inv_scale).cuda()

    def call(codes=None, scales=None):
        if kind == "fused":
            return kq.transform_quantize_mxfp4(A, fac, codes=codes, scales=scales)
        if kind == "smoothquant":
            return kq.smoothquant_quantize_mxfp4(A, inv, codes=codes, scales=scales)
        return kq.quantize_mxfp4(A, codes=codes, scales=scales)

    ref_c, ref_s = call()
    torch.cuda.synchronize()
    codes = torch.empty_like(ref_c)
    scales = torch.empty_like(ref_s)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(codes, scales)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(codes, scales)
    for rep in range(3):
        codes.zero_()
        scales.zero_()
        other_c, _ = kq.quantize_mxfp4(A)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, ref_c) and torch.equal(scales, ref_s), "replay %d" % rep
        assert other_c.shape == ref_c.shape


def test_empty_inputs(torch_dev, kq):
    torch = torch_dev
    case("empty inputs")
    A = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    c, s = kq.quantize_mxfp4(A)
    assert c.shape == (0, 128) and s.shape == (0, 8)
    c, s = kq.transform_quantize_mxfp4(A, torch.zeros((8, 5, 2, 2), device="cuda"))
    assert c.numel() == 0


# ---------------------------------------------------------------------------
# weight fold W T^{-T} and the fp32 quantizer on folded weights
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("o,d,seed", [(64, 256, 21), (3072, 3072, 1003)])
def test_inverse_fold(torch_dev, kq, orc, o, d, seed):
    torch = torch_dev
    case("fold o=%d d=%d" % (o, d))
    W = synth.weights(o, d, 1004)
    fac = synth.lu_perturbed_factors(d // 32, seed)
    Wf = kq.inverse_fold_weights(torch.from_numpy(W).cuda(), torch.from_numpy(fac).cuda())
    got = Wf.cpu().numpy().astype(np.float64)
    ref = orc.inverse_fold(W, fac)
    err = np.abs(got - ref).reshape(o, d // 32, 32).max(axis=2)
    nrm = np.sqrt((ref.reshape(o, d // 32, 32) ** 2).sum(axis=2))
    assert np.all(err <= 1e-5 * nrm)
    # the fp32 quantizer on the oracle's folded weights (rounded once to fp32)
    ref32 = ref.astype(np.float32)
    codes, scales = kq.quantize_mxfp4_f32(torch.from_numpy(ref32).cuda())
    c_ref, s_ref = orc.quantize_f32(ref32)
    assert np.array_equal(codes.cpu().numpy(), c_ref) and np.array_equal(scales.cpu().numpy(), s_ref)


# ---------------------------------------------------------------------------
# W4A4 GEMM on the quantizer's output (the downstream check of Eq. 2)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k,seed", [(37, 50, 96, 1), (130, 64, 256, 2), (16, 16, 128, 3)])
def test_mxfp4_gemm_ragged(torch_dev, kq, orc, m, n, k, seed):
    """Seeded random MXFP4 operands (any code byte, scales around 2^0); k not a multiple of 128."""
    torch = torch_dev
    case("mxfp4 gemm m=%d n=%d k=%d" % (m, n, k))
    rng = np.random.default_rng(seed)
    ca = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sa = rng.integers(118, 136, (m, k // 32), dtype=np.uint8)
    sw = rng.integers(118, 136, (n, k // 32), dtype=np.uint8)
    O = kq.mxfp4_gemm(*(torch.from_numpy(x).cuda() for x in (ca, sa, cw, sw)))
    ref = orc.gemm_dequant(ca, sa, cw, sw, k)
    got = O.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 1e-6, rel
    # every element to fp32 accumulation accuracy
    absdot = np.abs(orc.dequantize(ca, sa, k)) @ np.abs(orc.dequantize(cw, sw, k)).T
    assert np.all(np.abs(got - ref) <= 64 * 2.0 ** -24 * absdot + 1e-30)


def test_w4a4_downstream_flux(torch_dev, kq, orc):
    """The 18432x3072 FLUX activations through the fused path and the 3072x3072 weights
    through the fold and the fp32 quantizer, multiplied by the W4A4 GEMM: checked against
    the oracle's pipeline from the same seeded inputs on sampled rows (1e-3 relative
    Frobenius), the GEMM kernel alone on the oracle's operands, and the quantization
    error |Q(AT) Q(WT^-T)^T - A W^T| against T = I."""
    torch = torch_dev
    case("w4a4 downstream 18432x3072x3072")
    w = workload("flux_18432x3072")
    W = synth.weights(3072, 3072, 1004)
    fac = w.factors
    rows = sample_rows(w.m, 192, seed=5)
    A_dev = dev_bf16(torch, w.A)
    fac_dev = torch.from_numpy(fac).cuda()
    # GPU pipeline
    Wf = kq.inverse_fold_weights(torch.from_numpy(W).cuda(), fac_dev)
    cw_g, sw_g = kq.quantize_mxfp4_f32(Wf)
    ca_g, sa_g = kq.transform_quantize_mxfp4(A_dev, fac_dev)
    O_g = kq.mxfp4_gemm(ca_g, sa_g, cw_g, sw_g)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    kq.mxfp4_gemm(ca_g, sa_g, cw_g, sw_g, out=O_g)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    og = gather(torch, O_g, rows).astype(np.float64)
    # oracle pipeline from the seeded inputs
    A_rows = w.A[rows]
    ca_r, sa_r, _ = orc.transform_quantize(A_rows, fac, want_y=False)
    cw_r, sw_r = orc.quantize_f64(orc.inverse_fold(W, fac))
    O_r = orc.gemm_dequant(ca_r, sa_r, cw_r, sw_r, 3072)
    rel = np.linalg.norm(og - O_r) / np.linalg.norm(O_r)
    assert rel <= 1e-3, rel
    # the GEMM kernel alone on the oracle's operands
    O_k = kq.mxfp4_gemm(*(torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (ca_r, sa_r, cw_r, sw_r)))
    rel_k = np.linalg.norm(O_k.cpu().numpy().astype(np.float64) - O_r) / np.linalg.norm(O_r)
    assert rel_k < 1e-6, rel_k
    # quantization error with the transform vs T = I (and a block-Hadamard control)
    Af = synth.bf16_bits_to_f32(A_rows).astype(np.float64)
    exact = Af @ W.astype(np.float64).T
    ca_i, sa_i = orc.quantize_bf16(A_rows)
    cw_i, sw_i = orc.quantize_f32(W)
    err_i = np.linalg.norm(orc.gemm_dequant(ca_i, sa_i, cw_i, sw_i, 3072) - exact)
    err_t = np.linalg.norm(O_r - exact)
    hf = synth.hadamard_factors(96)
    ca_h, sa_h, _ = orc.transform_quantize(A_rows, hf, want_y=False)
    cw_h, sw_h = orc.quantize_f64(orc.inverse_fold(W, hf))
    err_h = np.linalg.norm(orc.gemm_dequant(ca_h, sa_h, cw_h, sw_h, 3072) - exact)
    err_g = np.linalg.norm(og - exact)
    print("[w4a4] rel(gpu pipeline vs oracle) %.3g, rel(gemm kernel) %.3g, |E| T=I %.4g, "
          "T=Kronecker %.4g (gpu %.4g), T=Hadamard %.4g, gemm %.1f us = %.1f TFLOP/s"
          % (rel, rel_k, err_i, err_t, err_g, err_h, ms * 1e3, 2 * 18432 * 3072 * 3072 / ms / 1e9),
          flush=True)
    # The error with the transform at the paper's Hadamard initialization is below T = I.
    # The workload's random, uncalibrated LU-perturbed factors are not expected to beat
    # T = I (reducing the error is what calibration does); their error is reported only.
    assert err_h < err_i
