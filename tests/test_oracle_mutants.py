"""The oracle's pins catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a wrong tie rule,
an off-by-one exponent, a reversed Kronecker bit order, a transposed operand,
a lost sign of zero, swapped nibbles, a wrong exponent clamp, a wrong
Hadamard sign, a lost normalization, a wrong group offset), builds it into a
temporary library on the CPU and checks that at least one of the pins in
test_oracle_pins.py fails against it. The shipped oracle is untouched.
"""
import os
import subprocess

import pytest

import oracle
import importlib.util

import tests.test_oracle_calib_pins as cpins
import tests.test_oracle_hadamard_pins as hpins
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kq_oracle.c")

MUTANTS = {
    "tie_to_odd": ("(dd == bestd && (i % 2) == 0)", "(dd == bestd && (i % 2) == 1)",
                   [pins.test_tie_table_from_golden]),
    "exponent_off_by_one": ("int e = (ex - 1) - 2;", "int e = (ex - 1) - 1;",
                            [pins.test_every_level_every_exponent_round_trips]),
    "clamp_at_minus_126": ("if (e < -127) e = -127;", "if (e < -126) e = -126;",
                           [pins.test_every_bf16_alone_in_a_block]),
    "kron_bit_order_reversed": ("int bit = 5 - k;", "int bit = k - 1;",
                                [pins.test_bit_order_g1_is_stride_16]),
    "fold_not_transposed": ("(double)w[r] * Ki[col * 32 + r]", "(double)w[r] * Ki[r * 32 + col]",
                            [lambda o: pins.test_invariance_eq1(o, "lu")]),
    "transform_transposed": ("a[r] * K[r * 32 + col]", "a[r] * K[col * 32 + r]",
                             [lambda o: pins.test_invariance_eq1(o, "lu")]),
    "sign_of_zero_lost": ("if (signbit(y[i])) code |= 8;", "if (y[i] < 0) code |= 8;",
                          [pins.test_zero_block_and_signed_zero]),
    "nibbles_swapped": ("(uint8_t)(code << ((i % 2) * 4))", "(uint8_t)(code << ((1 - i % 2) * 4))",
                        [pins.test_worked_examples_golden]),
    "inverse_sign_slip": ("Gi[k][0][1] = -G[k][0][1] / det;", "Gi[k][0][1] = G[k][0][1] / det;",
                          [pins.test_inverse_is_kron_of_inverses]),
    "hadamard_or_not_and": ("popcountll((unsigned long long)(r & col))",
                            "popcountll((unsigned long long)(r | col))",
                            [lambda o: hpins.test_matches_scipy_hadamard(o, 64)]),
    "hadamard_unnormalized": ("y[col] = s * inv_sqrt_n;", "y[col] = s;",
                              [lambda o: hpins.test_involution_and_norm(o, 256)]),
    "hadamard_group_offset": ("hadamard_group(x + g * c->n, c->n", "hadamard_group(x + g, c->n",
                              [hpins.test_groups_are_independent]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new, checks = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + old
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(mpath), "-o", str(so), "-lm"])
    mutant = oracle.Oracle(oracle.load(str(so)))
    caught = False
    for check in checks:
        try:
            check(mutant)
        except AssertionError:
            caught = True
    assert caught, "pins did not notice the planted mistake " + name


# Planted mistakes in the calibration oracle (oracle/calib.py): each mutated copy
# is loaded as a separate module and the finite-difference pin must reject it.
CALIB_SRC = os.path.join(os.path.dirname(oracle.__file__), "calib.py")
CALIB_MUTANTS = {
    "inverse_term_sign": ("dK = dK - KinvT @", "dK = dK + KinvT @"),
    "inverse_not_transposed": ("KinvT @ np.transpose(dP, (0, 2, 1)) @ KinvT", "KinvT @ dP @ KinvT"),
    "eq6_chain_sign": ("g00 + c * g10 + g11 / (a * a)", "g00 + c * g10 - g11 / (a * a)"),
    "regularizer_sign": ("- lam_A * 2.0 / (M * d) * (f[\"Xq\"] - f[\"X\"])",
                         "+ lam_A * 2.0 / (M * d) * (f[\"Xq\"] - f[\"X\"])"),
    "kron_bit_order": ("((r >> (4 - k)) & 1, (c >> (4 - k)) & 1)", "((r >> k) & 1, (c >> k) & 1)"),
}


@pytest.mark.parametrize("name", sorted(CALIB_MUTANTS))
def test_calibration_pins_catch_planted_mistake(name, tmp_path, orc):
    old, new = CALIB_MUTANTS[name]
    src = open(CALIB_SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + old
    path = tmp_path / "calib_mutant.py"
    path.write_text(src.replace(old, new).replace("from . import get as _get_oracle",
                                                  "from oracle import get as _get_oracle"))
    spec = importlib.util.spec_from_file_location("calib_mutant_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises(AssertionError):
        cpins.check_gradient(orc, mod, 2)


LOWRANK_SRC = os.path.join(os.path.dirname(oracle.__file__), "lowrank.py")
LOWRANK_MUTANTS = {
    "residual_sign": ("resid = Wt - L @ R", "resid = Wt + L @ R", "test_unquantized_layer_is_AW"),
    "no_bf16_rounding": ("Z = round_bf16(X) @ qdq(R, orc).T", "Z = X @ qdq(R, orc).T",
                         "test_grid_exact_branch_is_plain_product"),
}


@pytest.mark.parametrize("name", sorted(LOWRANK_MUTANTS))
def test_lowrank_pins_catch_planted_mistake(name, tmp_path, orc, monkeypatch):
    import tests.test_oracle_lowrank_pins as lpins
    old, new, pin = LOWRANK_MUTANTS[name]
    src = open(LOWRANK_SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + old
    path = tmp_path / "lowrank_mutant.py"
    path.write_text(src.replace(old, new).replace("from . import get as _get_oracle",
                                                  "from oracle import get as _get_oracle"))
    spec = importlib.util.spec_from_file_location("lowrank_mutant_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(lpins, "lowrank", mod)
    with pytest.raises(AssertionError):
        getattr(lpins, pin)(orc)
