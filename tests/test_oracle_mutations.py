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
    (pins.test_im2col_matches_torch_unfold, {}),
    (pins.test_im2col_hand_example, {}),
    (pins.test_conv_weight_gradient_is_g_rows_times_patches, {}),
    (pins.test_grad_rows_layout_and_scale, {}),
    (pins.test_grad_rows_bf16_rounding, {}),
    (pins.test_grad_matrix_concatenates_bias, {}),
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
    "im2col_taps_transposed": ("im2col", lambda x, kernel=(1, 1), stride=(1, 1), padding=(0, 0), dilation=(1, 1),
                               ones=False: _im2col_taps_transposed(x, kernel, stride, padding, dilation, ones)),
    "im2col_padding_dropped": ("im2col", lambda x, kernel=(1, 1), stride=(1, 1), padding=(0, 0), dilation=(1, 1),
                               ones=False: _REAL_IM2COL(x, kernel, stride, (0, 0), dilation, ones)),
    "grad_rows_no_transpose": ("grad_rows", lambda gy, scale, bf16=False: _grad_rows_no_transpose(gy, scale, bf16)),
    "grad_rows_scale_dropped": ("grad_rows", lambda gy, scale, bf16=False: _REAL_GRAD_ROWS(gy, 1.0, bf16)),
}

_REAL_IM2COL = oracle.im2col
_REAL_GRAD_ROWS = oracle.grad_rows


def _im2col_taps_transposed(x, kernel, stride, padding, dilation, ones):
    # columns in (c, j, i) order instead of (c, i, j)
    a = _REAL_IM2COL(x, kernel, stride, padding, dilation, False)
    n, c = a.shape[0], np.asarray(x).shape[1]
    a = a.reshape(n, c, kernel[0], kernel[1]).transpose(0, 1, 3, 2).reshape(n, -1)
    if ones:
        a = np.concatenate([a, np.ones((n, 1), dtype=a.dtype)], axis=1)
    return a


def _grad_rows_no_transpose(gy, scale, bf16):
    # rows read as [b*c] blocks of positions, i.e. the NCHW order kept
    g = _REAL_GRAD_ROWS(gy, scale, bf16)
    gy = np.asarray(gy)
    return g.reshape(gy.shape[0], -1, gy.shape[1]).transpose(0, 2, 1).reshape(g.shape)


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_python_mutation_is_caught(name, monkeypatch):
    attr, fn = PY_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    assert failing_pins(), f"planted mistake {name!r} was not caught by any pin"
