"""Pins of the low-rank layer oracle (oracle/lowrank.py; KroQuant Sec. 3.4 Eq. 11, App. D), no GPU.

- the bf16 rounding against torch's conversion of float32 values and a
  brute-force nearest search;
- Eq. 11 without quantization is A W^T (Eq. 1 plus the split W~ = (W~ - L R) + L R);
- L = R = 0 reduces the layer to the plain W4A4 product of the other oracle;
- L, R whose 32-blocks lie on the E2M1 grid (one entry of magnitude 4 * 2^e per
  block) quantize exactly, so the low-rank term is a plain matrix product.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import lowrank

LEVELS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_round_bf16_matches_torch_on_float32():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(lowrank.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_brute_force_nearest():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2000) * 3.0
    got = lowrank.round_bf16(x)
    for v, g in zip(x, got):
        _, e = np.frexp(v)
        step = 2.0 ** (e - 8)
        cands = np.floor(v / step) * step + np.array([0.0, step])
        dist = np.abs(cands - v)
        best = cands[np.argmin(dist)] if dist[0] != dist[1] else \
            cands[int(round(cands[1] / step)) % 2 == 0]  # tie: the even significand
        assert g == best


def layer_inputs(seed, M=48, d=64, o=40, r=32):
    rng = np.random.default_rng(seed)
    A_bits = synth.random_bf16_matrix(M, d, seed=seed)
    W = synth.weights(o, d, seed + 1)
    fac = synth.lu_perturbed_factors(d // 32, seed + 2)
    L = rng.standard_normal((o, r)) / np.sqrt(r)
    R = rng.standard_normal((r, d)) / np.sqrt(d)
    return A_bits, W, fac, L, R


def test_unquantized_layer_is_AW(orc):
    A_bits, W, fac, L, R = layer_inputs(3)
    O, _ = lowrank.layer(A_bits, W, fac, L, R, orc, quantize=False)
    A = synth.bf16_bits_to_f32(A_bits).astype(np.float64)
    ref = A @ W.astype(np.float64).T
    # fp32 factors: K and K^-1 are exact inverses of each other up to fp64 rounding
    assert np.allclose(O, ref, rtol=0, atol=1e-9 * np.abs(ref).max())


def test_zero_branch_is_plain_w4a4(orc):
    A_bits, W, fac, L, R = layer_inputs(4)
    L[:] = 0.0
    R[:] = 0.0
    O, parts = lowrank.layer(A_bits, W, fac, L, R, orc)
    ca, sa, _ = orc.transform_quantize(A_bits, fac, want_y=False)
    cw, sw = orc.quantize_f64(orc.inverse_fold(W, fac))
    ref = orc.gemm_dequant(ca, sa, cw, sw, A_bits.shape[1])
    assert np.array_equal(parts["Z"], np.zeros_like(parts["Z"]))
    assert np.allclose(O, ref, rtol=1e-14, atol=0)


def grid_matrix(rng, rows, cols):
    """Entries on the E2M1 grid times 2^e per 32-block, each block holding a +-4 2^e."""
    out = np.empty((rows, cols))
    for i in range(rows):
        for b in range(cols // 32):
            e = int(rng.integers(-6, 3))
            v = rng.choice(LEVELS, 32) * rng.choice([-1.0, 1.0], 32)
            v[int(rng.integers(32))] = 4.0 * rng.choice([-1.0, 1.0])
            out[i, 32 * b:32 * b + 32] = v * 2.0 ** e
    return out


def test_grid_exact_branch_is_plain_product(orc):
    A_bits, W, fac, _, _ = layer_inputs(5)
    rng = np.random.default_rng(5)
    L = grid_matrix(rng, W.shape[0], 32)
    R = grid_matrix(rng, 32, A_bits.shape[1])
    assert np.array_equal(lowrank.qdq(L, orc), L) and np.array_equal(lowrank.qdq(R, orc), R)
    _, parts = lowrank.layer(A_bits, W, fac, L, R, orc)
    X = orc.transform(A_bits, fac)
    want = (lowrank.round_bf16(X) @ R.T) @ L.T
    assert np.allclose(parts["low"], want, rtol=1e-13, atol=0)
