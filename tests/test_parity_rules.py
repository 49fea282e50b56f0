"""The fused-path comparison rules (tests/parity.py) applied to planted GPU results
on the CPU: a scale tie (the two block maxima straddle a power of two, so both
E8M0 scales are correct) is admitted only for a small share of the blocks, and
the codes it changes count toward the 1e-4 mismatch fraction.
"""
import numpy as np
import pytest

from tests import parity


def planted(orc, nblocks, ties, seed=0):
    """y_ref with block maxima just below 4 in `ties` blocks, y_gpu equal to y_ref
    except that those maxima are rounded up to exactly 4 (a relative change of
    2^-40, far inside rule 1), so their scale byte moves up by one."""
    rng = np.random.default_rng(seed)
    y_ref = rng.uniform(-3.0, 3.0, (1, nblocks * 32))
    y_ref[0, ::32] = 3.5
    y_gpu = y_ref.copy()
    for b in range(ties):
        y_ref[0, 32 * b] = 4.0 - 2.0 ** -38
        y_gpu[0, 32 * b] = 4.0
    codes_g, scales_g = orc.quantize_f64(y_gpu)
    return y_ref, y_gpu, codes_g, scales_g


def report(orc, y_ref, y_gpu, codes_g, scales_g):
    A = np.zeros(y_ref.shape, np.uint16)  # unused: y_ref is given
    return parity.fused_report(orc, A, None, codes_g, scales_g, y_gpu, y_ref=y_ref)


def test_one_scale_tie_in_many_blocks_passes(orc):
    y_ref, y_gpu, c, s = planted(orc, 20000, 1)
    rep = report(orc, y_ref, y_gpu, c, s)
    assert rep["scale_tie_blocks"] == 1
    assert rep["mismatches"] == 0 and rep["scale_tie_mismatches"] > 0


def test_many_scale_ties_fail(orc):
    y_ref, y_gpu, c, s = planted(orc, 20000, 50)
    with pytest.raises(AssertionError, match="scale-tie blocks"):
        report(orc, y_ref, y_gpu, c, s)


def test_scale_tie_codes_count_toward_the_fraction(orc):
    # the codes a tie changes are part of the reported (and limited) fraction
    y_ref, y_gpu, c, s = planted(orc, 20000, 2)
    rep = report(orc, y_ref, y_gpu, c, s)
    assert rep["scale_tie_blocks"] == 2 and rep["scale_tie_mismatches"] > 32
    assert rep["mismatch_frac"] == rep["scale_tie_mismatches"] / rep["elements"]


def test_scale_differing_without_a_straddle_fails(orc):
    y_ref, y_gpu, c, s = planted(orc, 100, 0)
    s = s.copy()
    s[0, 7] += 1
    with pytest.raises(AssertionError):
        report(orc, y_ref, y_gpu, c, s)
