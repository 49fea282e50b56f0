"""Comparison rules between the GPU path and the CPU oracle (test infrastructure).

Quantize-only, SmoothQuant and fp32 quantize: codes and scales bit-exact.

Fused transform + quantize (tolerances as the build states them):
  1. per block, max |y_gpu - y_ref| <= 1e-5 * ||y_ref||_2 (y_ref in float64);
  2. the GPU's codes and scales are the quantization of the GPU's own y: the
     scale byte follows max|y_gpu| and each code is the nearest-even E2M1 level
     of |y_gpu| / 2^e with the sign of y_gpu (codes 0x8 and 0x0 equivalent).
     This is checked here with numpy on the GPU's output; the oracle itself only
     ever sees the seeded inputs;
  3. against the oracle's quantization of y_ref: at most 1e-4 of the elements
     differ, each by at most one E2M1 level, and only where a rounding
     boundary lies between y_ref / 2^e and y_gpu / 2^e (a rounding tie). A
     block whose scale differs must be a scale tie: the two block maxima
     straddle a power of two. Such blocks are counted separately, and they
     are not free: every code of such a block that differs from the oracle's
     counts toward the 1e-4 mismatch fraction (rule 2 already pins each of
     them to the GPU's own y), and at most 1e-4 of the blocks may be scale ties.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-5
MISMATCH_FRAC = 1e-4
BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def unpack(codes: np.ndarray) -> np.ndarray:
    """[m][d/2] bytes -> [m][d] nibbles (element 2k is the low nibble)."""
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def zero_equiv(n: np.ndarray) -> np.ndarray:
    """Map -0 (0x8) to +0 (0x0)."""
    return np.where(n == 8, 0, n)


def assert_codes_equal_mod_signed_zero(c1, c2, what=""):
    a, b = zero_equiv(unpack(c1)), zero_equiv(unpack(c2))
    bad = np.argwhere(a != b)
    assert bad.size == 0, "%s: %d nibbles differ, first at %s" % (what, len(bad), bad[:5].tolist())


def expected_levels(v: np.ndarray) -> np.ndarray:
    """E2M1 magnitude index of v >= 0 (exact float64): count of rounding boundaries
    passed; at a boundary between levels i and i+1 the even one wins, i.e. ties at
    0.75, 1.75 and 3.5 go up and ties at 0.25, 1.25, 2.5 and 5 stay down."""
    idx = np.zeros(v.shape, dtype=np.int8)
    for i, b in enumerate(BOUNDS):
        up_on_tie = (i + 1) % 2 == 0
        idx += (v > b) | ((v == b) & up_on_tie)
    return idx


def check_self_consistent(codes_g, scales_g, y_g, rows_per_chunk=2048):
    """Rule 2 on the GPU's own y (numpy; no oracle call)."""
    m, d = y_g.shape
    nblk = d // 32
    for r0 in range(0, m, rows_per_chunk):
        y = y_g[r0:r0 + rows_per_chunk].astype(np.float64)
        mm = y.shape[0]
        yb = y.reshape(mm, nblk, 32)
        amax = np.abs(yb).max(axis=2)
        _, ex = np.frexp(amax)  # amax = f 2^ex, 0.5 <= f < 1, so floor(log2 amax) = ex - 1
        e = np.where(amax == 0, -127, np.clip(ex - 3, -127, 127))
        sg = scales_g[r0:r0 + mm]
        assert np.array_equal(sg.astype(np.int64), e + 127), "scale not implied by max|y_gpu|"
        v = np.abs(yb) * np.exp2(-e.astype(np.float64))[..., None]
        lvl = expected_levels(v).reshape(mm, d)
        sign = np.signbit(y).astype(np.int8) * 8
        want = np.where(lvl == 0, 0, lvl | sign)
        got = zero_equiv(unpack(codes_g[r0:r0 + mm]))
        bad = np.argwhere(got != want)
        assert bad.size == 0, "code not the quantization of y_gpu at %s" % (bad[:5] + [r0, 0]).tolist()


def fused_report(orc, A_rows, factors, codes_g, scales_g, y_g, y_ref=None):
    """Apply rules 1-3 to rows already gathered from a GPU run; returns stats."""
    m, d = A_rows.shape[0], y_g.shape[1]
    nblk = d // 32
    if y_ref is None:
        y_ref = orc.transform(A_rows, factors, d=d)
    yg = y_g.astype(np.float64)
    # rule 1
    yr_b = y_ref.reshape(m, nblk, 32)
    err = np.abs(yg.reshape(m, nblk, 32) - yr_b).max(axis=2)
    nrm = np.sqrt((yr_b ** 2).sum(axis=2))
    bad1 = err > REL_TOL * nrm
    assert not bad1.any(), "y error above 1e-5 * block norm in %d blocks; worst ratio %g" % (
        bad1.sum(), (err / np.maximum(nrm, 1e-300)).max())
    # rule 2
    check_self_consistent(codes_g, scales_g, y_g)
    # rule 3
    cr, sr = orc.quantize_f64(y_ref)
    scale_tie = sr != scales_g
    if scale_tie.any():
        ar = np.abs(yr_b).max(axis=2)[scale_tie]
        ag = np.abs(yg.reshape(m, nblk, 32)).max(axis=2)[scale_tie]
        lo, hi = np.minimum(ar, ag), np.maximum(ar, ag)
        p2 = 2.0 ** np.floor(np.log2(hi))
        assert np.all((lo < p2) & (p2 <= hi)), "scale differs without a power-of-two straddle"
    n_tie_blocks = int(scale_tie.sum())
    assert n_tie_blocks <= MISMATCH_FRAC * m * nblk, "%d scale-tie blocks of %d" % (n_tie_blocks, m * nblk)
    nr = zero_equiv(unpack(cr))
    ng = zero_equiv(unpack(codes_g))
    elem_tie = np.repeat(scale_tie, 32, axis=1)
    mism = (nr != ng) & ~elem_tie
    n_mis = int(mism.sum())
    n_tie_mis = int(((nr != ng) & elem_tie).sum())
    if n_mis:
        e = np.repeat(sr.astype(np.int64) - 127, 32, axis=1)[mism]
        vr = np.abs(y_ref[mism]) / 2.0 ** e
        vg = np.abs(yg[mism]) / 2.0 ** e
        lo, hi = np.minimum(vr, vg), np.maximum(vr, vg)
        tie_ok = ((BOUNDS[None, :] >= lo[:, None]) & (BOUNDS[None, :] <= hi[:, None])).any(axis=1)
        assert tie_ok.all(), "%d code mismatches not at a rounding boundary" % (~tie_ok).sum()
        same_sign = (nr[mism] & 8) == (ng[mism] & 8)
        lvl = np.abs((nr[mism] & 7).astype(int) - (ng[mism] & 7).astype(int))
        ok_level = (same_sign & (lvl <= 1)) | (~same_sign & ((nr[mism] & 7) + (ng[mism] & 7) <= 1))
        assert ok_level.all(), "a mismatch exceeds one E2M1 level"
    frac = (n_mis + n_tie_mis) / float(m * d)
    assert frac <= MISMATCH_FRAC, "mismatch fraction %g > 1e-4" % frac
    return {"elements": m * d, "mismatches": n_mis, "scale_tie_mismatches": n_tie_mis, "mismatch_frac": frac,
            "scale_tie_blocks": n_tie_blocks, "blocks": m * nblk,
            "max_err_over_norm": float((err / np.maximum(nrm, 1e-300)).max())}
