"""Pins of the comparison helpers through which every parity gate passes.

The GPU tests apply their tolerances with ``tests.gpu_helpers.rel_fro`` and
``upper_rel_fro``; the oracle carries ``rel_fro`` and ``rel_fro_upper`` for the
same purpose.  Each is the relative Frobenius error ||x - ref||_F / ||ref||_F
(the upper variants over the entries (i, j >= i), diagonal included).  The
values below are worked out by hand, so a comparator that returns zero, drops
the square root, divides by the wrong norm, takes the maximum entry instead of
the Frobenius norm, compares the wrong triangle or leaves out the diagonal
fails at least one of them (``test_planted_comparator_mistakes_are_caught``
plants each of those mistakes).
"""
import numpy as np
import pytest

import oracle
from tests import gpu_helpers

FULL = [gpu_helpers.rel_fro, oracle.rel_fro]
UPPER = [gpu_helpers.upper_rel_fro, oracle.rel_fro_upper]


def _ref3():
    # ||ref||_F = sqrt(4 + 1 + 4) = 3, all of it in row 0 (upper triangle)
    return np.array([[2.0, 1.0, 2.0],
                     [0.0, 0.0, 0.0],
                     [0.0, 0.0, 0.0]])


def pin_identical_is_zero(fn):
    ref = _ref3()
    assert fn(ref.copy(), ref) == 0.0


def pin_double_is_one(fn):
    ref = _ref3()
    assert fn(2.0 * ref, ref) == pytest.approx(1.0, rel=1e-15)


def pin_zero_is_one(fn):
    ref = _ref3()
    assert fn(np.zeros_like(ref), ref) == pytest.approx(1.0, rel=1e-15)


def pin_hand_3x3(fn):
    # one entry off by 1.5 on the diagonal: ||diff||_F = 1.5, ratio 1.5 / 3
    # (squared norms would give 0.25, the max-entry ratio 0.75)
    ref = _ref3()
    x = ref.copy()
    x[2, 2] += 1.5
    assert fn(x, ref) == pytest.approx(0.5, rel=1e-15)


def pin_hand_two_entries(fn):
    # two upper entries off by 2 and 4 (a 3-4-5 pattern scaled): ||diff||_F
    # = sqrt(4 + 16) = sqrt(20), relative to 3
    ref = _ref3()
    x = ref.copy()
    x[0, 1] -= 2.0
    x[1, 2] += 4.0
    assert fn(x, ref) == pytest.approx(np.sqrt(20.0) / 3.0, rel=1e-15)


def pin_float32_inputs_compared_in_float64(fn):
    # 1 + 2^-23 against 1 (exact in float32): the difference must survive;
    # ||ref||_F = sqrt(3), nothing below the diagonal
    ref = np.array([[1.0, 1.0], [0.0, 1.0]], dtype=np.float32)
    x = ref.copy()
    x[0, 0] = np.float32(1.0 + 2.0 ** -23)
    assert fn(x, ref) == pytest.approx(2.0 ** -23 / np.sqrt(3.0), rel=1e-12)


def pin_scale_invariant(fn):
    rng = np.random.default_rng(4)
    ref = rng.standard_normal((5, 5))
    x = ref + 1e-3 * rng.standard_normal((5, 5))
    assert fn(1e6 * x, 1e6 * ref) == pytest.approx(fn(x, ref), rel=1e-12)


def pin_full_sees_lower_and_order(fn):
    """Full comparators: a change in the strict lower triangle counts, and a
    transposed (non-symmetric) matrix is not equal to the original."""
    ref = _ref3()
    x = ref.copy()
    x[2, 0] = 3.0
    assert fn(x, ref) == pytest.approx(1.0, rel=1e-15)
    assert fn(ref.T, ref) == pytest.approx(np.sqrt(2 * 5.0) / 3.0, rel=1e-15)


def pin_upper_ignores_strict_lower(fn):
    """Upper comparators: the strict lower triangle of either argument is not
    looked at, the diagonal and the strict upper triangle are."""
    ref = _ref3()
    x = ref.copy()
    x[np.tril_indices(3, -1)] = 1e30
    r2 = ref.copy()
    r2[np.tril_indices(3, -1)] = -7.0
    assert fn(x, r2) == 0.0
    d = ref.copy()
    d[1, 1] = 3.0
    assert fn(d, ref) == pytest.approx(1.0, rel=1e-15)
    u = ref.copy()
    u[0, 2] = -1.0
    assert fn(u, ref) == pytest.approx(1.0, rel=1e-15)


COMMON = [pin_identical_is_zero, pin_double_is_one, pin_zero_is_one, pin_hand_3x3, pin_hand_two_entries,
          pin_float32_inputs_compared_in_float64, pin_scale_invariant]
FULL_PINS = COMMON + [pin_full_sees_lower_and_order]
UPPER_PINS = COMMON + [pin_upper_ignores_strict_lower]


@pytest.mark.parametrize("fn", FULL, ids=["gpu_helpers.rel_fro", "oracle.rel_fro"])
@pytest.mark.parametrize("pin", FULL_PINS, ids=lambda p: p.__name__)
def test_full_comparator(fn, pin):
    pin(fn)


@pytest.mark.parametrize("fn", UPPER, ids=["gpu_helpers.upper_rel_fro", "oracle.rel_fro_upper"])
@pytest.mark.parametrize("pin", UPPER_PINS, ids=lambda p: p.__name__)
def test_upper_comparator(fn, pin):
    pin(fn)


# ------------------------------------------------------- planted mistakes --

def _f(x):
    return np.asarray(x, dtype=np.float64)


def _upper(fn):
    def g(x, ref):
        iu = np.triu_indices(np.asarray(ref).shape[0])
        return fn(np.asarray(x)[iu], np.asarray(ref)[iu])
    return g


FULL_MUTANTS = {
    "always_zero": lambda x, ref: 0.0,
    "squared_norms": lambda x, ref: float(np.sum((_f(x) - _f(ref)) ** 2) / np.sum(_f(ref) ** 2)),
    "normalised_by_x": lambda x, ref: float(np.linalg.norm(_f(x) - _f(ref)) / np.linalg.norm(_f(x))),
    "max_entry": lambda x, ref: float(np.abs(_f(x) - _f(ref)).max() / np.abs(_f(ref)).max()),
    "absolute_error": lambda x, ref: float(np.linalg.norm(_f(x) - _f(ref))),
    "compares_transpose": lambda x, ref: float(np.linalg.norm(_f(x).T - _f(ref)) / np.linalg.norm(_f(ref))),
    "difference_of_norms": lambda x, ref: float(abs(np.linalg.norm(_f(x)) - np.linalg.norm(_f(ref))) /
                                                np.linalg.norm(_f(ref))),
    "half_precision": lambda x, ref: float(np.linalg.norm(np.asarray(x, np.float16).astype(np.float64) -
                                                          np.asarray(ref, np.float16).astype(np.float64)) /
                                           np.linalg.norm(_f(ref))),
    "upper_only": _upper(lambda x, ref: float(np.linalg.norm(_f(x) - _f(ref)) / np.linalg.norm(_f(ref)))),
}

UPPER_MUTANTS = {
    "always_zero": lambda x, ref: 0.0,
    "lower_triangle": lambda x, ref: gpu_helpers.rel_fro(_f(x)[np.tril_indices(_f(ref).shape[0])],
                                                         _f(ref)[np.tril_indices(_f(ref).shape[0])]),
    "strict_upper": lambda x, ref: gpu_helpers.rel_fro(_f(x)[np.triu_indices(_f(ref).shape[0], 1)],
                                                       _f(ref)[np.triu_indices(_f(ref).shape[0], 1)]),
    "whole_matrix": lambda x, ref: gpu_helpers.rel_fro(x, ref),
    "squared_norms": _upper(FULL_MUTANTS["squared_norms"]),
    "normalised_by_x": _upper(FULL_MUTANTS["normalised_by_x"]),
    "max_entry": _upper(FULL_MUTANTS["max_entry"]),
}


def _caught(fn, pins):
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except Exception:                       # noqa: BLE001 -- any failure counts
            return True
    return False


@pytest.mark.parametrize("name", sorted(FULL_MUTANTS))
def test_planted_full_comparator_mistakes_are_caught(name):
    assert _caught(FULL_MUTANTS[name], FULL_PINS), name


@pytest.mark.parametrize("name", sorted(UPPER_MUTANTS))
def test_planted_upper_comparator_mistakes_are_caught(name):
    assert _caught(UPPER_MUTANTS[name], UPPER_PINS), name
