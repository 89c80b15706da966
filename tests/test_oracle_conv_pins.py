"""Pins of the fp64 conv1d oracle (oracle/conv1d.py), on the CPU.

Each check states what the pages and the mathematics fix, not a retyped copy of
the oracle's loop: a tap on the current token is the identity, a tap one token
back is a shift that takes its first value from the state (the orientation of
PyTorch's left-padded Conv1d, Candle page "Bug elimination log", bug 2), a
library convolution (torch.nn.functional.conv1d, fp64) agrees on a random case,
a sequence split in two with the state carried equals the whole (prefix reuse,
NPU page "New in v2"), a packed batch equals separate runs, the L2-normalised
heads have unit norm and ignore scale, v is untouched.  Planted mistakes (a
reversed kernel, a reversed state, a window off by one, a dropped state, the
norm over the wrong span) are each caught by at least one check.
"""
import numpy as np
import pytest
import torch

from oracle.conv1d import causal_conv1d, conv_qkv, l2_normalise_heads

C, K = 6, 4


def _case(seed, T=11, n_state=1):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, C)), rng.standard_normal((C, K)), rng.standard_normal((n_state, C, K - 1))


def check_identity_tap(fn):
    x, _, s = _case(1)
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    y, ns = fn(x, w, None, s)
    np.testing.assert_array_equal(y, x)
    np.testing.assert_array_equal(ns[0], x[-(K - 1):].T)


def check_shift_tap_reads_state(fn):
    x, _, s = _case(2)
    w = np.zeros((C, K))
    w[:, K - 2] = 1.0                                        # one token back
    y, _ = fn(x, w, None, s)
    np.testing.assert_array_equal(y[1:], x[:-1])
    np.testing.assert_array_equal(y[0], s[0, :, K - 2])      # the newest state entry
    w = np.zeros((C, K))
    w[:, 0] = 1.0                                            # K - 1 tokens back: the oldest state entry
    y, _ = fn(x, w, None, s)
    np.testing.assert_array_equal(y[0], s[0, :, 0])
    np.testing.assert_array_equal(y[K - 1:], x[:-(K - 1)])


def check_against_torch_conv1d(fn):
    x, w, _ = _case(3, T=17)
    y, _ = fn(x, w, None, None)
    xt = torch.tensor(x.T[None])                             # [1, C, T]
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (K - 1, 0)), torch.tensor(w[:, None, :]),
                                     groups=C)[0].numpy().T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def check_split_with_state_equals_whole(fn):
    x, w, s = _case(4, T=13)
    y, ns = fn(x, w, None, s)
    for cut in (1, 2, 5, 12):
        y1, s1 = fn(x[:cut], w, None, s)
        y2, s2 = fn(x[cut:], w, None, s1)
        np.testing.assert_array_equal(np.concatenate([y1, y2]), y)
        np.testing.assert_array_equal(s2, ns)


def check_packed_equals_separate(fn):
    rng = np.random.default_rng(5)
    lengths = [4, 1, 0, 7]
    x = rng.standard_normal((sum(lengths), C))
    w = rng.standard_normal((C, K))
    s = rng.standard_normal((len(lengths), C, K - 1))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    y, ns = fn(x, w, cu, s)
    for i in range(len(lengths)):
        yi, si = fn(x[cu[i]:cu[i + 1]], w, None, s[i:i + 1])
        np.testing.assert_array_equal(y[cu[i]:cu[i + 1]], yi)
        np.testing.assert_array_equal(ns[i], si[0])


CHECKS = [check_identity_tap, check_shift_tap_reads_state, check_against_torch_conv1d,
          check_split_with_state_equals_whole, check_packed_equals_separate]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(causal_conv1d)


def _generic(x, w, cu, state, variant):
    """A hand-written conv with one planted mistake (for the mutation checks)."""
    x, w = np.asarray(x, float), np.asarray(w, float)
    T, Cc = x.shape
    Kk = w.shape[1]
    cu = np.array([0, T]) if cu is None else np.asarray(cu)
    n = len(cu) - 1
    s = np.zeros((n, Cc, Kk - 1)) if state is None else np.asarray(state, float)
    y = np.zeros((T, Cc))
    ns = np.zeros((n, Cc, Kk - 1))
    for i in range(n):
        a, b = cu[i], cu[i + 1]
        st = s[i][:, ::-1] if variant == "reversed_state" else s[i]
        if variant == "dropped_state":
            st = np.zeros_like(st)
        xs = np.concatenate([st.T, x[a:b]], 0)
        ww = w[:, ::-1] if variant == "reversed_kernel" else w
        off = 1 if variant == "off_by_one" else 0
        for t in range(b - a):
            acc = np.zeros(Cc)
            for j in range(Kk):
                idx = t + j - off
                if 0 <= idx < xs.shape[0]:
                    acc += ww[:, j] * xs[idx]
            y[a + t] = acc
        ns[i] = xs[xs.shape[0] - (Kk - 1):].T
    return y, ns


@pytest.mark.parametrize("variant", ["reversed_kernel", "reversed_state", "off_by_one", "dropped_state"])
def test_checks_catch_planted_mistakes(variant):
    caught = 0
    for check in CHECKS:
        try:
            check(lambda x, w, cu, s: _generic(x, w, cu, s, variant))
        except AssertionError:
            caught += 1
    assert caught >= 1, variant


def test_silu_option():
    x, _, s = _case(6)
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    y, _ = causal_conv1d(x, w, None, s, silu=True)
    np.testing.assert_allclose(y, x * 0.5 * (1.0 + np.tanh(0.5 * x)), rtol=1e-13, atol=1e-15)


def test_qkv_split_and_head_norms():
    rng = np.random.default_rng(7)
    hqk, hv, dk, dv = 2, 4, 8, 4
    Cc = 2 * hqk * dk + hv * dv
    x = rng.standard_normal((9, Cc))
    w = rng.standard_normal((Cc, K))
    q, k, v, _ = conv_qkv(x, w, hqk, hv, dk, dv, eps=0.0)
    y, _ = causal_conv1d(x, w)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_array_equal(v.reshape(9, -1), y[:, 2 * hqk * dk:])
    # each head's direction is the conv output's: q * |y_head| = y_head
    yq = y[:, :hqk * dk].reshape(9, hqk, dk)
    np.testing.assert_allclose(q * np.linalg.norm(yq, axis=-1, keepdims=True), yq, rtol=1e-12, atol=1e-14)
    # a mistake in the span of the norm (whole q block instead of per head) is visible
    wrong = l2_normalise_heads(y[:, :hqk * dk], hqk * dk, 0.0).reshape(9, hqk, dk)
    assert not np.allclose(np.linalg.norm(wrong, axis=-1), 1.0)


def _norm_variants(y, head_dim, eps, variant):
    """l2_normalise_heads with a planted mistake in where eps enters (for the pin below)."""
    h = np.asarray(y, dtype=np.float64).reshape(y.shape[0], -1, head_dim)
    ss = np.sum(h * h, axis=-1, keepdims=True)
    den = {"outside_root": np.sqrt(ss) + eps, "squared": np.sqrt(ss + eps * eps),
           "dropped": np.sqrt(ss)}[variant]
    return (h / den).reshape(y.shape)


def check_head_norm_eps_closed_form(fn):
    """A constant head of value c over d components with eps inside the root: every component
    becomes c / sqrt(d c^2 + eps) (c = 0.5, d = 4, eps = 0.25: 0.5 / sqrt(1.25))."""
    d, c, eps = 4, 0.5, 0.25
    y = np.full((3, 2 * d), c)
    out = fn(y, d, eps)
    np.testing.assert_allclose(out, np.full_like(y, c / np.sqrt(d * c * c + eps)), rtol=1e-15)
    # zero heads stay zero (eps keeps the division finite)
    np.testing.assert_array_equal(fn(np.zeros((2, d)), d, eps), np.zeros((2, d)))


def test_head_norm_eps_closed_form():
    check_head_norm_eps_closed_form(l2_normalise_heads)


@pytest.mark.parametrize("variant", ["outside_root", "squared", "dropped"])
def test_head_norm_eps_pin_catches_planted_mistakes(variant):
    with pytest.raises(AssertionError):
        check_head_norm_eps_closed_form(lambda y, d, eps: _norm_variants(y, d, eps, variant))


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        causal_conv1d(np.ones((3, 4)), np.ones((5, 2)))
    with pytest.raises(ValueError):
        causal_conv1d(np.ones((3, 4)), np.ones((4, 3)), None, np.ones((1, 4, 3)))
