"""Pins of the fp64 gated-RMSNorm oracle (oracle/output_norm.py), on the CPU.

Each check states a property fixed by the mathematics of the norm as read from
the pages (scale invariance of the norm, NPU page "How it works"; eps inside the
mean square, Candle page "Bug elimination log", bug 7), not a retyped copy of
the oracle's formula: closed forms for constant rows, an independent route
through the Euclidean norm and a tanh form of the gate, sign and per-row
independence.  The same checks are then run against planted mistakes (eps
outside the root, a sum instead of a mean, sigmoid instead of silu, the norm
over the wrong axis, the weight on the wrong axis), each of which must fail at
least one of them.
"""
import numpy as np
import pytest

from oracle.output_norm import gated_rmsnorm

DV = 16


def _case(seed, rows=6, dv=DV):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((rows, 3, dv)) * np.array([0.01, 1.0, 50.0])[None, :, None]
    z = rng.standard_normal((rows, 3, dv)) * 2.0
    w = rng.uniform(0.5, 1.5, dv)
    return o, z, w


def _gate_tanh(z):
    # silu(z) = z * sigmoid(z) = z * (1 + tanh(z / 2)) / 2
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def check_scale_invariance(fn):
    o, z, w = _case(1)
    for a in (1e-3, 7.0, 1e4):
        np.testing.assert_allclose(fn(a * o, z, w, 0.0), fn(o, z, w, 0.0), rtol=1e-12, atol=0)


def check_constant_rows_closed_form(fn):
    # a row of equal entries c has mean square c^2: the norm gives c / sqrt(c^2 + eps)
    for c in (0.3, -2.0, 5.0):
        for eps in (1e-6, 1.0):
            o = np.full((2, DV), c)
            z = np.full((2, DV), 40.0)            # silu(40) = 40 to fp64 precision
            w = np.ones(DV)
            want = c / np.sqrt(c * c + eps) * 40.0
            np.testing.assert_allclose(fn(o, z, w, eps), want, rtol=1e-13, atol=0)


def check_euclidean_route(fn):
    # eps = 0: o / rms(o) = sqrt(dv) o / |o|_2, and the gate through tanh
    o, z, w = _case(2)
    want = np.sqrt(DV) * o / np.linalg.norm(o, axis=-1, keepdims=True) * w * _gate_tanh(z)
    np.testing.assert_allclose(fn(o, z, w, 0.0), want, rtol=1e-12, atol=1e-15)


def check_zero_gate(fn):
    o, z, w = _case(3)
    assert np.all(fn(o, np.zeros_like(z), w, 1e-6) == 0.0)


def check_sign_and_rows(fn):
    o, z, w = _case(4)
    y = fn(o, z, w, 1e-6)
    np.testing.assert_allclose(fn(-o, z, w, 1e-6), -y, rtol=0, atol=0)
    # every (token, head) row on its own: rescaling one row leaves the others unchanged
    o2 = o.copy()
    o2[1, 2] *= 1e3
    y2 = fn(o2, z, w, 0.0)
    mask = np.ones(o.shape[:2], bool)
    mask[1, 2] = False
    np.testing.assert_allclose(y2[mask], fn(o, z, w, 0.0)[mask], rtol=1e-13, atol=0)


def check_weight_per_column(fn):
    o, z, _ = _case(5)
    e3 = np.zeros(DV)
    e3[3] = 1.0
    y = fn(o, z, e3, 1e-6)
    assert np.all(y[..., np.arange(DV) != 3] == 0.0)
    assert np.all(y[..., 3] != 0.0)


CHECKS = [check_scale_invariance, check_constant_rows_closed_form, check_euclidean_route, check_zero_gate,
          check_sign_and_rows, check_weight_per_column]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(gated_rmsnorm)


# planted mistakes: each must be caught by at least one check
def _mut_eps_outside(o, z, w, eps):
    return o / (np.sqrt(np.mean(o * o, -1, keepdims=True)) + eps) * w * z / (1 + np.exp(-z))


def _mut_sum(o, z, w, eps):
    return o / np.sqrt(np.sum(o * o, -1, keepdims=True) + eps) * w * z / (1 + np.exp(-z))


def _mut_sigmoid(o, z, w, eps):
    return o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps) * w / (1 + np.exp(-z))


def _mut_axis(o, z, w, eps):
    return o / np.sqrt(np.mean(o * o, -2, keepdims=True) + eps) * w * z / (1 + np.exp(-z))


def _mut_weight_axis(o, z, w, eps):
    return o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps) * np.mean(w) * z / (1 + np.exp(-z))


def _mut_no_gate(o, z, w, eps):
    return o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps) * w * z


@pytest.mark.parametrize("mutant", [_mut_eps_outside, _mut_sum, _mut_sigmoid, _mut_axis, _mut_weight_axis,
                                    _mut_no_gate], ids=lambda m: m.__name__)
def test_checks_catch_planted_mistakes(mutant):
    caught = 0
    for check in CHECKS:
        try:
            check(mutant)
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, "no check caught %s" % mutant.__name__


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        gated_rmsnorm(np.ones((2, 4)), np.ones((2, 5)), np.ones(4))
    with pytest.raises(ValueError):
        gated_rmsnorm(np.ones((2, 4)), np.ones((2, 4)), np.ones(3))
