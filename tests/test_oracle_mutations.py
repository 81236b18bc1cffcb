"""Planted mistakes in the oracle must be caught by its pins.

Each case plants one plausible mistake (a dropped term, a wrong sign or index,
a transposed operand, a missing scale) into a private copy of the oracle --
the C source is edited as text and compiled to a temporary library, Python
functions are swapped in -- and asserts that at least one pin in
``test_oracle_pins`` fails.  The real oracle is never modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import oracle.build as obuild
from tests import test_oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

PIN_CASES = [
    (pins.test_factor_brute_force_exact, dict(rows=5, d=8)),
    (pins.test_factor_trace_closed_form, {}),
    (pins.test_factor_bias_column_closed_form, {}),
    (pins.test_factor_symmetric_psd, {}),
    (pins.test_running_average_limits, {}),
    (pins.test_running_average_three_steps_closed_form, {}),
    (pins.test_pack_literal, dict(golden_dir=GOLDEN)),
    (pins.test_pack_size_closed_form, {}),
    (pins.test_pack_unpack_round_trip_bits, {}),
    (pins.test_pack_adjoint, {}),
    (pins.test_inverse_residual, dict(d=64, gamma=1e-3)),
    (pins.test_inverse_zero_matrix, {}),
    (pins.test_inverse_two_by_two, {}),
    (pins.test_inverse_sherman_morrison, dict(c=0.3, d=33, gamma=0.01)),
    (pins.test_cholesky_recovers_known_factor, {}),
    (pins.test_inverse_info_first_failing_pivot, dict(k=5)),
    (pins.test_precondition_kronecker_brute_force, dict(da=16, dg=16)),
    (pins.test_precondition_kronecker_brute_force, dict(da=9, dg=2)),
    (pins.test_precondition_closed_forms, {}),
]


def failing_pins():
    failed = []
    for fn, kw in PIN_CASES:
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:                       # noqa: BLE001 -- any failure counts
            failed.append(fn.__name__)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert failing_pins() == []


C_MUTATIONS = {
    "pack_drops_diagonal": ("for (int64_t j = i; j < dl; ++j) packed[p++]", "for (int64_t j = i + 1; j < dl; ++j) packed[p++]"),
    "unpack_no_mirror": ("m[l][j * dl + i] = v;", "(void)0;"),
    "cholesky_wrong_sign": ("yi[j] -= uki * uk[j];", "yi[j] += uki * uk[j];"),
    "cholesky_wrong_index": ("yi[j] -= uki * uk[j];", "yi[j] -= uki * uk[i];"),
    "forward_solve_wrong_index": ("w[i] -= uk[i] * wk;", "w[i] -= uk[k] * wk;"),
    "back_solve_dropped_term": ("s -= ui[k] * z[k];", "s -= 0.0 * z[k];"),
    "damping_dropped": ("y[i * d + i] += gamma;", "y[i * d + i] += 0.0 * gamma;"),
    "info_off_by_one": ("return k + 1;", "return k;"),
    "pivot_not_checked": ("if (!(p > 0.0) || !isfinite(p)) return k + 1;", "if (0) return k + 1;"),
}


@pytest.mark.parametrize("name", sorted(C_MUTATIONS))
def test_c_mutation_is_caught(name, tmp_path, monkeypatch):
    old, new = C_MUTATIONS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = tmp_path / "mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mutated), "-o", str(lib), "-lm"],
                   check=True, capture_output=True)
    real = oracle._load()
    mlib = ctypes.CDLL(str(lib))
    for fname in ("oracle_packed_size", "oracle_pack", "oracle_unpack", "oracle_cholesky_upper",
                  "oracle_damped_inverse", "oracle_damped_inverse_columns"):
        getattr(mlib, fname).restype = getattr(real, fname).restype
        getattr(mlib, fname).argtypes = getattr(real, fname).argtypes
    monkeypatch.setattr(oracle, "_lib", mlib)
    assert failing_pins(), f"planted mistake {name!r} was not caught by any pin"


def _f64(x):
    return np.asarray(x, dtype=np.float64)


PY_MUTATIONS = {
    "factor_missing_scale": ("factor", lambda x: _f64(x).T @ _f64(x)),
    "factor_wrong_operand_order": ("factor", lambda x: (_f64(x) @ _f64(x).T)[: _f64(x).shape[1], : _f64(x).shape[1]] / _f64(x).shape[0]),
    "running_average_swapped_weights": ("running_average",
                                        lambda m, f, eps, first: _f64(f).copy() if first else (1 - eps) * _f64(m) + eps * _f64(f)),
    "precondition_missing_right_inverse": ("precondition", lambda zg, g, za: _f64(zg) @ _f64(g)),
    "precondition_swapped_inverses": ("precondition", lambda zg, g, za: _f64(za) @ _f64(g) @ _f64(zg)),
}


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_python_mutation_is_caught(name, monkeypatch):
    attr, fn = PY_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    assert failing_pins(), f"planted mistake {name!r} was not caught by any pin"
