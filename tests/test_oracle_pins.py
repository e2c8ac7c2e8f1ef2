"""Pins of the CPU oracle (the checks live in ``oracle_checks.py``).

The pages print no worked numeric example, so the oracle is pinned by closed
forms, invariants, exact-rational brute force, the online identity and an
independent library routine; see ``oracle_checks.py`` for each pin's source.
"""

import pytest

import oracle
import oracle_checks as C


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def test_p1_rows_sum_to_one(orc):
    C.check_p1_rows_sum_to_one(orc)


def test_p2_identical_keys(orc):
    C.check_p2_identical_keys(orc)


def test_p3_constant_v(orc):
    C.check_p3_constant_v(orc)


def test_p4_online_equals_direct_every_split(orc):
    C.check_p4_online_equals_direct_every_split(orc)


def test_p4_online_kernel_tiles_peaked(orc):
    C.check_p4_online_kernel_tiles_peaked(orc)


def test_p5_single_key(orc):
    C.check_p5_single_key(orc)


def test_p5_two_keys_logistic(orc):
    C.check_p5_two_keys_logistic(orc)


def test_p5_exact_rational(orc):
    C.check_p5_exact_rational(orc)


def test_p6_zero_scale(orc):
    C.check_p6_zero_scale(orc)


def test_p7_key_shift(orc):
    C.check_p7_key_shift(orc)


def test_p8_permutations(orc):
    C.check_p8_permutations(orc)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_p9_library_crosscheck(orc, cfg):
    C.check_p9_library_crosscheck(orc, cfg)


def test_p9_small_sampled(orc):
    C.check_p9_small_sampled(orc)


def test_p10_peaked_limit(orc):
    C.check_p10_peaked_limit(orc)


def test_rejects_bad_arguments(orc):
    C.check_rejects_bad_arguments(orc)


def test_bf16_widening_is_exact(orc):
    C.check_bf16_widening_is_exact(orc)


def test_golden_exact_rational(orc):
    C.check_golden_exact_rational(orc)


@pytest.mark.parametrize("check", C.SOFTMAX_CHECKS, ids=lambda f: f.__name__[6:])
def test_softmax_pins(orc, check):
    check(orc)


@pytest.mark.parametrize("check", C.RMSNORM_CHECKS, ids=lambda f: f.__name__[6:])
def test_rmsnorm_pins(orc, check):
    check(orc)
