"""Pins for the row-softmax oracle, checked against facts that do not come from the oracle.

As for the attention oracle, each pin is a function of the oracle callable, and
`test_pins_catch_planted_mistakes` re-runs them with one step of the oracle replaced by a
plausible slip; every slip must fail at least one pin.

Sources of the pinned facts:
  * the hand-derived closed forms in tests/golden/softmax_cases.json;
  * closed forms and invariants of the softmax: rows sum to one, a single column gets weight
    one, a constant row is uniform with lse = c*x + ln C, shift invariance (lse shifts by the
    scaled shift), scale folding, permutation equivariance;
  * a pure-Python scalar loop on tiny inputs (brute force, math.exp, no max shift);
  * SciPy's softmax and logsumexp, the textbook library routines;
  * the online recurrence with several block sizes ("Tri Dao: prediction", transcript: the
    row is split into pieces that are rescaled and still give the right answer).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle.softmax as OS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "softmax_cases.json")
TOL = 1e-12


def _num(s):
    s = str(s)
    if "+ln(" in s:
        a, b = s.split("+ln(")
        return float(Fraction(a)) + math.log(float(Fraction(b[:-1])))
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def _arr(rows):
    return np.array([[_num(x) for x in r] for r in rows], dtype=np.float64)


def sm():
    """The oracle entry point, looked up at call time so planted mistakes take effect."""
    return OS.softmax_rows_fp64


def _rand(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---- pins ---------------------------------------------------------------------------------

def pin_golden():
    for case in json.load(open(GOLDEN))["cases"]:
        x = _arr(case["x"])
        y, lse = sm()(x, scale=_num(case["scale"]))
        np.testing.assert_allclose(y, _arr(case["y"]), rtol=0, atol=TOL, err_msg=case["name"])
        if "exp_lse" in case:
            np.testing.assert_allclose(np.exp(lse), [_num(e) for e in case["exp_lse"]], rtol=TOL, atol=0,
                                       err_msg=case["name"])
        else:
            np.testing.assert_allclose(lse, [_num(e) for e in case["lse"]], rtol=TOL, atol=TOL, err_msg=case["name"])


def pin_rows_sum_to_one():
    x = _rand(1, 5, 37, scale=3.0)
    y, _ = sm()(x, scale=0.7)
    assert (y >= 0).all()
    np.testing.assert_allclose(y.sum(axis=-1), 1.0, atol=1e-14)


def pin_single_column():
    x = _rand(2, 6, 1, scale=10.0)
    y, lse = sm()(x, scale=-0.3)
    np.testing.assert_array_equal(y, 1.0)
    np.testing.assert_allclose(lse, -0.3 * x[:, 0], atol=1e-13)


def pin_constant_row():
    C = 13
    x = np.full((3, C), 2.5)
    y, lse = sm()(x, scale=0.4)
    np.testing.assert_allclose(y, 1.0 / C, atol=1e-15)
    np.testing.assert_allclose(lse, 0.4 * 2.5 + math.log(C), atol=1e-14)


def pin_shift():
    x = _rand(3, 4, 29)
    t = np.array([[3.0], [-7.0], [100.0], [0.25]])
    y, lse = sm()(x, scale=0.5)
    y2, lse2 = sm()(x + t, scale=0.5)
    np.testing.assert_allclose(y2, y, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 0.5 * t[:, 0], atol=1e-12)


def pin_scale_folding():
    x = _rand(4, 3, 21)
    y, lse = sm()(x, scale=1.75)
    y2, lse2 = sm()(1.75 * x, scale=1.0)
    np.testing.assert_allclose(y, y2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


def pin_permutation():
    x = _rand(5, 2, 17)
    perm = np.random.default_rng(6).permutation(17)
    y, lse = sm()(x, scale=0.9)
    y2, lse2 = sm()(x[:, perm], scale=0.9)
    np.testing.assert_allclose(y2, y[:, perm], atol=1e-15)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)


def pin_brute_force():
    x = _rand(7, 3, 6)
    c = 0.8
    y, lse = sm()(x, scale=c)
    for r in range(3):
        e = [math.exp(c * float(v)) for v in x[r]]
        z = sum(e)
        for j in range(6):
            assert abs(y[r, j] - e[j] / z) <= 1e-14
        assert abs(lse[r] - math.log(z)) <= 1e-13


def pin_scipy():
    x = _rand(8, 7, 50, scale=4.0)
    y, lse = sm()(x, scale=1.3)
    np.testing.assert_allclose(y, scipy.special.softmax(1.3 * x, axis=-1), atol=1e-14)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(1.3 * x, axis=-1), atol=1e-12)


def pin_online():
    x = _rand(9, 4, 70, scale=5.0)
    y, lse = sm()(x, scale=0.6)
    for block in (1, 3, 16, 64, 100):
        y2, lse2 = OS.softmax_online_fp64(x, scale=0.6, block=block)
        np.testing.assert_allclose(y2, y, atol=1e-13, err_msg=f"block {block}")
        np.testing.assert_allclose(lse2, lse, atol=1e-12, err_msg=f"block {block}")


def pin_masked_entries():
    """-inf entries take weight zero and do not change the other weights."""
    x = _rand(10, 2, 9)
    xm = x.copy()
    xm[:, [2, 5]] = -np.inf
    keep = [0, 1, 3, 4, 6, 7, 8]
    y, lse = sm()(xm, scale=1.1)
    y2, lse2 = sm()(x[:, keep], scale=1.1)
    assert (y[:, [2, 5]] == 0).all()
    np.testing.assert_allclose(y[:, keep], y2, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


PINS = [pin_golden, pin_rows_sum_to_one, pin_single_column, pin_constant_row, pin_shift, pin_scale_folding,
        pin_permutation, pin_brute_force, pin_scipy, pin_online, pin_masked_entries]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


def test_accepts_bf16_torch_tensors():
    import torch

    x = torch.randn(3, 40, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    y, lse = OS.softmax_rows_fp64(x, scale=0.5)
    y2, lse2 = OS.softmax_rows_fp64(x.float().numpy(), scale=0.5)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(lse, lse2)


# ---- planted mistakes: every one must trip at least one pin --------------------------------

MUTANTS = {
    "scale_dropped": ("_scaled", lambda x, c: x),
    "scale_squared": ("_scaled", lambda x, c: c * c * x),
    "max_wrong_axis": ("_row_max", lambda s: s.max(axis=0, keepdims=True)),
    "max_not_subtracted": ("_exp_shifted", lambda s, m: np.exp(s)),
    "exp2_not_exp": ("_exp_shifted", lambda s, m: np.exp2(s - m)),
    "sum_wrong_axis": ("_row_sum", lambda e: e.sum(axis=0, keepdims=True)),
    "unnormalised": ("_normalise", lambda e, l: e),
    "lse_without_max": ("_lse", lambda m, l: np.log(l)[..., 0]),
    "lse_log2": ("_lse", lambda m, l: (m + np.log2(l))[..., 0]),
    "lse_of_max_only": ("_lse", lambda m, l: m[..., 0]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OS, attr, fn)
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ValueError):
            caught += 1
    assert caught >= 1, f"planted mistake {name} passed every pin"
