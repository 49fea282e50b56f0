"""Pins of the oracle's block-Hadamard baseline (no GPU).

The transform is the normalized Hadamard matrix of order n = 2^k applied to
each group of n consecutive channels: KroQuant Sec. 3.2 "Hadamard
initialization" defines H_n as the k-fold Kronecker power of
[[1,1],[1,-1]]/sqrt(2); Sec. 1 and Sec. 4.4 use it as the fixed-rotation
baseline at n = 32 (Table 2) and at n = d (the FWHT of Table 3). Each pin ties
the oracle to something outside it: scipy's Hadamard matrix, the closed form of
Sylvester's construction, the Kronecker recursion, the involution and norm
invariants, the hand-derived worked example, and the separately pinned
Kronecker oracle at n = 32.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def blockdiag_hadamard(x, n):
    """Reference product by scipy's (unnormalized) Sylvester matrix, group by group."""
    H = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
    m, d = x.shape
    return (x.reshape(m, d // n, n) @ H).reshape(m, d)


@pytest.mark.parametrize("n", [1, 2, 4, 32, 64, 512, 1024])
def test_matches_scipy_hadamard(orc, n):
    x = np.random.default_rng(n).standard_normal((5, 2 * n))
    y = orc.hadamard_f64(x, n)
    ref = blockdiag_hadamard(x, n)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(x).sum(axis=1).max()


def test_unit_vectors_give_sylvester_entries_exactly(orc):
    n = 64  # 1/sqrt(64) = 1/8: every entry exact
    y = orc.hadamard_f64(np.eye(n), n)
    r = np.arange(n)[:, None]
    c = np.arange(n)[None, :]
    parity = np.vectorize(lambda v: bin(v).count("1") & 1)(r & c)
    assert np.array_equal(y, np.where(parity == 1, -0.125, 0.125))


def test_kronecker_recursion(orc):
    """H_2n = H_2 (x) H_n: the top channel bit is the first Kronecker factor."""
    n = 128
    x = np.random.default_rng(3).standard_normal((4, 2 * n))
    y2 = orc.hadamard_f64(x, 2 * n)
    lo = orc.hadamard_f64(x[:, :n], n)
    hi = orc.hadamard_f64(x[:, n:], n)
    want = np.concatenate([lo + hi, lo - hi], axis=1) / np.sqrt(2.0)
    assert np.abs(y2 - want).max() <= 1e-13 * np.abs(x).sum(axis=1).max()


@pytest.mark.parametrize("n", [32, 256, 2048])
def test_involution_and_norm(orc, n):
    x = np.random.default_rng(7).standard_normal((3, 2 * n))
    y = orc.hadamard_f64(x, n)
    back = orc.hadamard_f64(y, n)
    assert np.abs(back - x).max() <= 1e-12 * np.abs(x).max() * np.log2(n)
    ny = np.sqrt((y.reshape(3, 2, n) ** 2).sum(axis=2))
    nx = np.sqrt((x.reshape(3, 2, n) ** 2).sum(axis=2))
    assert np.allclose(ny, nx, rtol=1e-13)


def test_groups_are_independent(orc):
    n = 64
    x = np.random.default_rng(11).standard_normal((2, 3 * n))
    y = orc.hadamard_f64(x, n)
    x2 = x.copy()
    x2[:, n:2 * n] *= -3.0
    y2 = orc.hadamard_f64(x2, n)
    assert np.array_equal(y[:, :n], y2[:, :n]) and np.array_equal(y[:, 2 * n:], y2[:, 2 * n:])
    scale = np.abs(x2[:, n:2 * n]).sum(axis=1, keepdims=True)
    assert (np.abs(y2[:, n:2 * n] + 3.0 * y[:, n:2 * n]) <= 1e-14 * scale).all()


def test_bf16_entry_widens_exactly(orc):
    A = synth.random_bf16_matrix(6, 256, seed=5)
    _, _, y = orc.hadamard_quantize(A, 128)
    x = synth.bf16_bits_to_f32(A).astype(np.float64)
    assert np.array_equal(y, orc.hadamard_f64(x, 128))


def test_worked_example_hadamard32_from_golden(orc):
    ex = [e for e in json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["examples"]
          if e["transform"] == "hadamard"][0]
    blk = np.zeros(32, dtype=np.float32)
    for k, v in ex["block"].items():
        blk[int(k)] = v
    A = synth.to_bf16_bits(blk.astype(np.float64))[None, :]
    codes, scales, _ = orc.hadamard_quantize(A, 32)
    assert int(scales[0, 0]) == ex["expect_scale_byte"]
    out = np.empty(32, dtype=np.uint8)
    out[0::2], out[1::2] = codes[0] & 15, codes[0] >> 4
    for c in range(32):
        ch = int(list(ex["block"])[0])
        want = 7 | (8 if bin(ch & c).count("1") & 1 else 0)
        assert out[c] == want, c


def test_hadamard32_agrees_with_kronecker_oracle(orc):
    """At n = 32 the baseline is K = H32/sqrt(32), i.e. Eq. 12 with every factor the
    Hadamard 2x2; the Kronecker oracle carries those factors in fp32 (1/sqrt(2)
    rounded), so the two agree to a few fp32 units of the row's scale."""
    rec = synth.recipe("tiny_64x256", 64)
    A = rec.generate()
    d = A.shape[1]
    _, _, yh = orc.hadamard_quantize(A, 32)
    yk = orc.transform(A, synth.hadamard_factors(d // 32))
    x = np.abs(synth.bf16_bits_to_f32(A).astype(np.float64)).reshape(64, d // 32, 32).sum(axis=2)
    err = np.abs(yh - yk).reshape(64, d // 32, 32).max(axis=2)
    assert (err <= 4e-7 * x + 1e-300).all()


def test_full_width_constant_row(orc):
    """All-ones row: H_n 1 / sqrt(n) = sqrt(n) e_0, exactly (sums of +-1)."""
    n = 1024
    A = np.full((2, n), 0x3F80, dtype=np.uint16)  # bf16 1.0
    codes, scales, y = orc.hadamard_quantize(A, n)
    want = np.zeros(n)
    want[0] = 32.0
    assert np.array_equal(y[0], want) and not np.signbit(y[0]).any()
    assert scales[0, 0] == 130 and (scales[0, 1:] == 0).all()  # 32 = 4 * 2^3
    assert codes[0, 0] == 6 and (codes[0, 1:] == 0).all()


def test_rejects_bad_group_size(orc):
    A = np.zeros((1, 96), dtype=np.uint16)
    for n in (3, 48, 64):
        with pytest.raises(ValueError):
            orc.hadamard_quantize(A, n)
