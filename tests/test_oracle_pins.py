"""Pins of the CPU oracle against what the KroQuant paper and mathematics fix.

None of these checks retypes the oracle's own formula: each compares it with a
closed form, a library routine (numpy.kron, numpy.linalg, exact fractions), a
brute-force enumeration or a value derived by hand from the paper
(arXiv 2607.21446v1). They run on the CPU.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LEVELS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
          Fraction(4), Fraction(6)]


def popcount(x):
    return bin(x).count("1")


def sylvester32():
    return np.array([[(-1) ** popcount(r & c) for c in range(32)] for r in range(32)], float)


def kron_chain(G):
    K = np.array([[1.0]])
    for k in range(5):
        K = np.kron(K, G[k].astype(np.float64))
    return K


def butterfly_reshape(x, G):
    """y = x K by contracting each index bit of a (2,2,2,2,2) view (G1 on the top bit)."""
    t = x.reshape(x.shape[:-1] + (2, 2, 2, 2, 2)).astype(np.float64)
    for k in range(5):
        axis = t.ndim - 5 + k
        t = np.moveaxis(np.tensordot(t, G[k].astype(np.float64), axes=([axis], [0])), -1, axis)
    return t.reshape(x.shape)


# --------------------------------------------------------------------------
# Kronecker blocks: Sec. 3.2 Eq. 5, Sec. 3.5.1 Eq. 12, Hadamard initialization
# --------------------------------------------------------------------------

def test_hadamard_factors_give_sylvester_h32(orc):
    f = synth.hadamard_factors(1)[0]
    K = orc.block_K(f)
    ref = sylvester32() / math.sqrt(32.0)
    # the ABI carries fp32 1/sqrt(2); five of them multiply to 2^-2.5 within 5 fp32 ulps
    assert np.max(np.abs(K - ref)) <= 6 * 2.0 ** -24 * (1 / math.sqrt(32))
    assert np.allclose(K, K.T, atol=0, rtol=0)
    assert np.allclose(K @ K.T, np.eye(32), atol=1e-6)
    assert abs(np.linalg.det(K) - 1.0) < 1e-5


def test_hadamard_exact_factors_float64(orc):
    # fp32 factors that are exact (+-0.5) give an exactly scaled Sylvester matrix: G = 2^-1/2 * H2 * 2^-1/2
    f = np.array([[0.5, 0.5], [0.5, -0.5]], np.float32)
    K = orc.block_K(np.broadcast_to(f, (5, 2, 2)))
    assert np.array_equal(K, sylvester32() * 2.0 ** -5)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_eq5_eq12_numpy_kron_and_butterfly_agree(orc, seed):
    G = synth.lu_perturbed_factors(4, seed)
    for j in range(4):
        K12 = orc.block_K(G[j])
        K5 = orc.block_K_kron(G[j])
        Knp = kron_chain(G[j])
        assert np.max(np.abs(K12 - Knp)) < 1e-14 * np.max(np.abs(Knp))
        assert np.max(np.abs(K5 - Knp)) < 1e-14 * np.max(np.abs(Knp))
        x = np.random.default_rng(seed).standard_normal((7, 32))
        assert np.allclose(x @ K12, butterfly_reshape(x, G[j]), rtol=0, atol=1e-13)


def test_bit_order_g1_is_stride_16(orc):
    # G1 = swap, others identity: K is the permutation c -> c xor 16 (Eq. 12, bit 4 for k = 1)
    G = synth.special_factors(1, "identity")[0]
    G[0] = [[0, 1], [1, 0]]
    K = orc.block_K(G)
    P = np.zeros((32, 32))
    for r in range(32):
        P[r, r ^ 16] = 1
    assert np.array_equal(K, P)
    G = synth.special_factors(1, "identity")[0]
    G[4] = [[0, 1], [1, 0]]
    K = orc.block_K(G)
    P = np.zeros((32, 32))
    for r in range(32):
        P[r, r ^ 1] = 1
    assert np.array_equal(K, P)


def test_unit_determinant_and_det_k(orc):
    G = synth.lu_perturbed_factors(16, 7).astype(np.float64)
    dets = np.linalg.det(G)
    assert np.all(np.abs(np.abs(dets) - 1) < 2e-6)  # fp32 rounding of unit-|det| factors
    for j in range(16):
        K = orc.block_K(G[j])
        # det(A (x) B) = det(A)^n det(B)^m, so det K = prod det(G_k)^16
        assert np.isclose(np.linalg.det(K), np.prod(dets[j] ** 16), rtol=1e-9)
    assert abs(np.linalg.det(orc.block_K(synth.hadamard_factors(1)[0])) - 1) < 1e-5


def test_eq6_lu_parametrization(orc):
    rng = np.random.default_rng(5)
    abc = rng.standard_normal((6, 5, 3))
    abc[..., 0] += np.sign(abc[..., 0]) * 0.5  # keep a away from 0
    G = orc.factors_from_lu(abc)
    a, b, c = abc[..., 0], abc[..., 1], abc[..., 2]
    L = np.zeros(G.shape); L[..., 0, 0] = 1; L[..., 1, 0] = c; L[..., 1, 1] = 1
    U = np.zeros(G.shape); U[..., 0, 0] = a; U[..., 0, 1] = b; U[..., 1, 1] = -1 / a
    assert np.allclose(G, L @ U, rtol=1e-15, atol=1e-15)
    assert np.allclose(np.linalg.det(G), -1.0, atol=1e-12)
    # (a, b, c) = (cos pi/4, sin pi/4, 1) is the Hadamard initialization G^(0)
    h = orc.factors_from_lu(np.array([[[math.cos(math.pi / 4), math.sin(math.pi / 4), 1.0]] * 5]))
    g0 = np.array([[math.cos(math.pi / 4), math.sin(math.pi / 4)],
                   [math.sin(math.pi / 4), -math.cos(math.pi / 4)]])
    assert np.allclose(h[0, 0], g0, atol=1e-15)


def test_inverse_is_kron_of_inverses(orc):
    G = synth.lu_perturbed_factors(8, 11)
    for j in range(8):
        K = orc.block_K(G[j])
        Ki = orc.block_Kinv(G[j])
        assert np.max(np.abs(K @ Ki - np.eye(32))) < 1e-12
        assert np.allclose(Ki, np.linalg.inv(K), rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# Eq. 1 invariance: (A T)(W T^{-T})^T = A W^T
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["lu", "hadamard"])
def test_invariance_eq1(orc, kind):
    m, d, o = 64, 256, 48
    A = synth.workload("tiny_64x256").A
    fac = synth.lu_perturbed_factors(d // 32, 21) if kind == "lu" else synth.hadamard_factors(d // 32)
    W = synth.weights(o, d, 1004)
    AT = orc.transform(A, fac)
    Wf = orc.inverse_fold(W, fac)
    Af = synth.bf16_bits_to_f32(A).astype(np.float64)
    ref = Af @ W.astype(np.float64).T
    got = AT @ Wf.T
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 1e-4
    assert rel < 1e-12  # fp64 throughout: far below the 1e-4 bar
    # the transform side really is A T with T = diag(K^(j)) (Eq. 4)
    Tfull = np.zeros((d, d))
    for j in range(d // 32):
        Tfull[32 * j:32 * j + 32, 32 * j:32 * j + 32] = kron_chain(fac[j])
    assert np.allclose(AT, Af @ Tfull, rtol=1e-13, atol=1e-9)
    assert np.allclose(Wf, W.astype(np.float64) @ np.linalg.inv(Tfull).T, rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------------------
# MXFP4 quantizer (Sec. 3.1, Sec. 4.1, Appendix D)
# --------------------------------------------------------------------------

def nearest_even_level(v: Fraction) -> int:
    """Brute force: index of the nearest E2M1 level, ties to the even index."""
    dist = [abs(v - L) for L in LEVELS]
    best = min(dist)
    cands = [i for i, x in enumerate(dist) if x == best]
    return cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]


def floor_log2_fraction(x: Fraction) -> int:
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    if Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def test_e2m1_levels(orc):
    assert [orc.e2m1_value(c) for c in range(16)] == \
        [0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6]
    assert math.copysign(1, orc.e2m1_value(8)) == -1


def test_tie_table_from_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    for v, code in g["ties"]["v_to_code"]:
        assert orc.e2m1_round_index(v) == code
        assert nearest_even_level(Fraction(v)) == code
        lo, hi = np.nextafter(v, 0), np.nextafter(v, 10)
        assert orc.e2m1_round_index(lo) == nearest_even_level(Fraction(lo))
        assert orc.e2m1_round_index(hi) == nearest_even_level(Fraction(hi))


def test_round_index_brute_force_dense_grid(orc):
    # every multiple of 1/64 in [0, 8) plus the neighbours of every midpoint
    vals = [k / 64 for k in range(512)]
    for a, b in zip(LEVELS[:-1], LEVELS[1:]):
        mid = float((a + b) / 2)
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, 10)]
    vals += [6.0, 6.5, 7.0, 7.99, np.nextafter(8.0, 0)]
    for v in vals:
        assert orc.e2m1_round_index(v) == nearest_even_level(Fraction(v)), v


def test_every_level_every_exponent_round_trips(orc):
    # block max 4*2^e or 6*2^e pins the shared exponent at e; every level must decode exactly
    for e in range(-127, 126):
        for top in (4.0, 6.0):
            y = np.zeros(32)
            for i in range(16):
                y[i] = float(LEVELS[i % 8]) * 2.0 ** e
                y[16 + i] = -float(LEVELS[(i + 3) % 8]) * 2.0 ** e
            y[31] = top * 2.0 ** e
            codes, scale = orc.quantize_block(y)
            assert scale == e + 127
            deq = orc.dequantize(codes[None, :], np.array([[scale]], np.uint8), 32)[0]
            assert np.array_equal(deq, y)


def test_every_bf16_alone_in_a_block(orc):
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite].astype(np.uint16)
    n = bits.size
    A = np.zeros((n, 32), dtype=np.uint16)
    A[:, 5] = bits
    codes, scales = orc.quantize_bf16(A)
    x = synth.bf16_bits_to_f32(bits).astype(np.float64)
    ax = np.abs(x)
    mant, ex = np.frexp(ax)
    e_exp = np.where(ax == 0, -127, np.maximum(ex - 1 - 2, -127))
    assert np.array_equal(scales[:, 0].astype(int), e_exp + 127)
    code5 = (codes[:, 2] >> 4).astype(int)
    big = ax >= 2.0 ** -125
    v = ax[big] / 2.0 ** e_exp[big]               # exact, in [4, 8)
    assert np.all((v >= 4) & (v < 8))
    exp_big = np.where(v <= 5, 6, 7) | np.where(np.signbit(x[big]), 8, 0)
    assert np.array_equal(code5[big], exp_big)
    # tiny magnitudes: e clamps at -127 and v = |x| 2^127 < 4 is rounded normally
    for xb, cb in zip(x[~big], code5[~big]):
        v = Fraction(abs(xb)) * Fraction(2) ** 127
        assert cb == nearest_even_level(v) | (8 if math.copysign(1, xb) < 0 else 0)
    # every other element is +0 -> code 0
    others = np.delete(codes, 2, axis=1)
    assert not others.any()
    assert not (codes[:, 2] & 0x0F).any()


def test_brute_force_random_blocks_round_trip(orc):
    rng = np.random.default_rng(3)
    for _ in range(300):
        e = int(rng.integers(-127, 126))
        idx = rng.integers(0, 8, 32)
        sign = rng.integers(0, 2, 32)
        idx[rng.integers(0, 32)] = rng.choice([6, 7])
        y = np.array([(-1.0) ** s * float(LEVELS[i]) * 2.0 ** e for s, i in zip(sign, idx)])
        codes, scale = orc.quantize_block(y)
        assert scale == e + 127
        deq = orc.dequantize(codes[None, :], np.array([[scale]], np.uint8), 32)[0]
        assert np.array_equal(deq, y)
        # the sign bit follows y including -0 (level 0 with a minus sign)
        got = np.array([(codes[i // 2] >> (4 * (i % 2))) & 15 for i in range(32)])
        assert np.array_equal(got, idx | (sign * 8))


def test_general_blocks_against_fraction_brute_force(orc):
    rng = np.random.default_rng(9)
    for _ in range(200):
        y = rng.standard_normal(32) * 10.0 ** rng.uniform(-5, 5)
        y[rng.integers(0, 32)] *= rng.uniform(1, 100)
        codes, scale = orc.quantize_block(y)
        amax = max(Fraction(abs(v)) for v in y)
        e = max(floor_log2_fraction(amax) - 2, -127)
        assert scale == e + 127
        for i, v in enumerate(y):
            want = nearest_even_level(Fraction(abs(v)) / Fraction(2) ** e) | (8 if v < 0 else 0)
            assert (codes[i // 2] >> (4 * (i % 2))) & 15 == want


def test_zero_block_and_signed_zero(orc):
    codes, scale = orc.quantize_block(np.zeros(32))
    assert scale == 0 and not codes.any()
    y = np.zeros(32)
    y[0] = -0.0
    y[1] = 1.0
    y[2] = -1e-30
    codes, scale = orc.quantize_block(y)
    assert codes[0] & 15 == 8          # -0 keeps its sign
    assert (codes[1] & 15) == 8        # tiny negative rounds to -0
    assert scale == 127 - 2


def test_worked_examples_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    for ex in g["examples"]:
        A = np.zeros((1, 32), np.uint16)
        for ch, val in ex["block"].items():
            A[0, int(ch)] = synth.to_bf16_bits(np.array([val]))[0]
        if ex["transform"] == "identity":
            codes, scales = orc.quantize_bf16(A)
        else:
            codes, scales, _ = orc.transform_quantize(A, synth.hadamard_factors(1))
        assert scales[0, 0] == ex["expect_scale_byte"]
        got = [(codes[0, c // 2] >> (4 * (c % 2))) & 15 for c in range(32)]
        if "expect_codes" in ex:
            for c in range(32):
                assert got[c] == ex["expect_codes"].get(str(c), ex["expect_other_code"])
        else:
            for c in range(32):
                assert got[c] == 7 | (8 if popcount(3 & c) % 2 else 0)


def test_quantize_paths_agree_on_exact_inputs(orc):
    A = synth.workload("tiny_64x256").A
    c1, s1 = orc.quantize_bf16(A)
    X = synth.bf16_bits_to_f32(A)
    c2, s2 = orc.quantize_f32(X)
    c3, s3 = orc.quantize_f64(X.astype(np.float64))
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)
    assert np.array_equal(s1, s2) and np.array_equal(s1, s3)
    # lda > d: only the first d columns are read
    Apad = np.concatenate([A, np.full((64, 64), 0x7F00, np.uint16)], axis=1)
    c4, s4 = orc.quantize_bf16(Apad, d=256)
    assert np.array_equal(c1, c4) and np.array_equal(s1, s4)


def test_identity_transform_equals_quantize_only(orc):
    A = synth.workload("tiny_64x256").A
    for kind in ["identity", "swap", "signflip", "pow2", "mixed"]:
        f = synth.special_factors(8, kind)
        c, s, y = orc.transform_quantize(A, f)
        # the exact transform of a bf16 block by these factors is a signed, scaled permutation
        Kf = [orc.block_K(f[j]) for j in range(8)]
        X = synth.bf16_bits_to_f32(A).astype(np.float64)
        Y = np.concatenate([X[:, 32 * j:32 * j + 32] @ Kf[j] for j in range(8)], axis=1)
        assert np.array_equal(y, Y)
        c2, s2 = orc.quantize_f64(Y)
        assert np.array_equal(c, c2) and np.array_equal(s, s2)
        if kind == "identity":
            c3, s3 = orc.quantize_bf16(A)
            assert np.array_equal(c, c3) and np.array_equal(s, s3)


def test_smoothquant_is_one_fp32_multiply(orc):
    w = synth.workload("tiny_64x256")
    inv = w.inv_scale
    c, s = orc.smoothquant_quantize(w.A, inv)
    X = synth.bf16_bits_to_f32(w.A)
    Y = (X * inv[None, :]).astype(np.float32)  # numpy float32 multiply: IEEE, round to nearest
    c2, s2 = orc.quantize_f32(Y)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_smoothquant_scale_vector():
    w = synth.workload("tiny_64x256")
    X = np.abs(synth.bf16_bits_to_f32(w.A).astype(np.float64))
    want = (1.0 / np.sqrt(X.max(axis=0))).astype(np.float32)
    assert np.array_equal(w.inv_scale, want)


def test_dequantize_and_gemm(orc):
    rng = np.random.default_rng(1)
    ca = rng.integers(0, 256, (5, 32), dtype=np.uint8)
    sa = rng.integers(110, 140, (5, 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (3, 32), dtype=np.uint8)
    sw = rng.integers(110, 140, (3, 2), dtype=np.uint8)
    da = orc.dequantize(ca, sa, 64)
    dw = orc.dequantize(cw, sw, 64)
    # decode one element by hand: low nibble first
    b = int(ca[2, 7])
    sc = 2.0 ** (int(sa[2, 0]) - 127)
    assert da[2, 14] == float(LEVELS[b & 7]) * (-1.0) ** ((b >> 3) & 1) * sc
    assert da[2, 15] == float(LEVELS[(b >> 4) & 7]) * (-1.0) ** (b >> 7) * sc
    O = orc.gemm_dequant(ca, sa, cw, sw, 64)
    assert np.array_equal(O, da @ dw.T) or np.allclose(O, da @ dw.T, rtol=1e-15, atol=0)
    O2 = orc.gemm_dequant(ca, sa, cw, sw, 64, rows=[4, 1])
    assert np.array_equal(O2, O[[4, 1]])


def test_parity_rule2_levels_match_oracle(orc):
    """The test-side level rule used on GPU output agrees with the oracle's quantizer."""
    from tests import parity
    vals = np.array([k / 64 for k in range(512)] + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.9])
    vals = np.concatenate([vals, np.nextafter(vals, 0), np.nextafter(vals, 10)])
    got = parity.expected_levels(vals)
    want = np.array([orc.e2m1_round_index(v) for v in vals])
    assert np.array_equal(got, want)
