"""Pins of the float64 token shift and output gate (no GPU).

The token shift and the gate are pinned against what they do not compute themselves: the
library sigmoid (scipy.special.expit), the mu = 1 / mu = 0 extremes, the continuation of a
sequence from its last token, the adjoint identity of a linear map, and central finite
differences of the losses they define.
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import wkv_backward_direct, wkv_direct
from oracle.wkv_mix import (
    sigmoid,
    token_shift,
    token_shift_backward,
    wkv_gated,
    wkv_gated_backward,
    wkv_gated_backward_recurrent,
    wkv_gated_recurrent,
)


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(0.0, scale, shape)


def test_sigmoid_matches_library_and_saturates():
    r = np.concatenate([np.linspace(-40, 40, 801), [-1000.0, -745.0, 0.0, 745.0, 1000.0]])
    np.testing.assert_allclose(sigmoid(r), expit(r), rtol=1e-14, atol=1e-300)  # a few ulps
    assert sigmoid(np.array([0.0]))[0] == 0.5
    assert np.all(np.isfinite(sigmoid(np.array([-1e308, 1e308]))))
    np.testing.assert_allclose(sigmoid(-r) + sigmoid(r), 1.0, rtol=0, atol=1e-15)


def test_token_shift_extremes():
    x = rand((2, 7, 5), 0)
    prev = rand((2, 5), 1)
    mu = np.stack([np.ones(5), np.zeros(5), np.full(5, 0.5)])
    out = token_shift(x, mu, prev)
    np.testing.assert_array_equal(out[0], x)  # mu = 1: the current token
    np.testing.assert_array_equal(out[1][:, 1:], x[:, :-1])  # mu = 0: the previous token
    np.testing.assert_array_equal(out[1][:, 0], prev)
    np.testing.assert_allclose(out[2][:, 1:], 0.5 * (x[:, 1:] + x[:, :-1]), rtol=1e-15)
    # a fresh sequence has nothing before it
    np.testing.assert_array_equal(token_shift(x, mu)[1][:, 0], 0.0)


def test_token_shift_continues_a_split_sequence():
    x = rand((3, 12, 4), 2)
    mu = np.random.default_rng(3).uniform(0, 1, (3, 4))
    full = token_shift(x, mu)
    first = token_shift(x[:, :5], mu)
    second = token_shift(x[:, 5:], mu, x[:, 4])
    np.testing.assert_allclose(np.concatenate([first, second], axis=2), full, rtol=0, atol=1e-15)


def test_token_shift_backward_is_the_adjoint():
    """<g, S(x, prev)> = <gx, x> + <gprev, prev> for the linear map S at fixed mu."""
    x = rand((2, 9, 6), 4)
    prev = rand((2, 6), 5)
    mu = np.random.default_rng(6).uniform(-0.5, 1.5, (3, 6))
    g = rand((3, 2, 9, 6), 7)
    gx, _, gprev = token_shift_backward(x, mu, g, prev)
    lhs = float((g * token_shift(x, mu, prev)).sum())
    rhs = float((gx * x).sum() + (gprev * prev).sum())
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def test_token_shift_mu_gradient_by_differences():
    x = rand((2, 6, 3), 8)
    prev = rand((2, 3), 9)
    mu = np.random.default_rng(10).uniform(0, 1, (2, 3))
    g = rand((2, 2, 6, 3), 11)
    _, gmu, _ = token_shift_backward(x, mu, g, prev)
    h = 1e-3  # the map is linear in mu: central differences are exact up to rounding
    for m in range(2):
        for c in range(3):
            mp, mm = mu.copy(), mu.copy()
            mp[m, c] += h
            mm[m, c] -= h
            fd = ((g * token_shift(x, mp, prev)).sum() - (g * token_shift(x, mm, prev)).sum()) / (2 * h)
            assert abs(fd - gmu[m, :, c].sum()) < 1e-9


def test_gate_limits():
    w = np.exp(np.random.default_rng(12).uniform(-3, 1, 4))
    u = rand(4, 13, 0.5)
    k, v = rand((2, 10, 4), 14), rand((2, 10, 4), 15)
    y = wkv_direct(w, u, k, v)
    np.testing.assert_allclose(wkv_gated(w, u, k, v, np.full(k.shape, 60.0)), y, rtol=1e-15)
    np.testing.assert_allclose(wkv_gated(w, u, k, v, np.zeros(k.shape)), 0.5 * y, rtol=1e-15)
    assert np.all(np.abs(wkv_gated(w, u, k, v, np.full(k.shape, -800.0))) < 1e-300)


def test_gated_backward_by_differences():
    rng = np.random.default_rng(16)
    B, T, C = 2, 5, 3
    w = np.exp(rng.uniform(-3, 1, C))
    u = rng.normal(0, 0.5, C)
    k, v, r, gz = (rng.normal(0, 1.5, (B, T, C)) for _ in range(4))
    gw, gu, gk, gv, gr = wkv_gated_backward(w, u, k, v, r, gz)
    h = 1e-6

    def loss(**kw):
        a = {"w": w, "u": u, "k": k, "v": v, "r": r}
        a.update(kw)
        return float((gz * wkv_gated(a["w"], a["u"], a["k"], a["v"], a["r"])).sum())

    for name, grad in (("k", gk), ("v", gv), ("r", gr)):
        base = {"k": k, "v": v, "r": r}[name]
        for idx in np.ndindex(B, T, C):
            p, m = base.copy(), base.copy()
            p[idx] += h
            m[idx] -= h
            fd = (loss(**{name: p}) - loss(**{name: m})) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7, (name, idx)
    for name, grad in (("w", gw), ("u", gu)):
        base = {"w": w, "u": u}[name]
        for c in range(C):
            p, m = base.copy(), base.copy()
            p[c] += h
            m[c] -= h
            fd = (loss(**{name: p}) - loss(**{name: m})) / (2 * h)
            assert abs(fd - grad[:, c].sum()) < 1e-7, (name, c)


def test_open_gate_backward_is_the_plain_backward():
    rng = np.random.default_rng(17)
    w = np.exp(rng.uniform(-3, 1, 4))
    u = rng.normal(0, 0.5, 4)
    k, v, gz = (rng.normal(0, 1, (2, 8, 4)) for _ in range(3))
    got = wkv_gated_backward(w, u, k, v, np.full(k.shape, 60.0), gz)
    ref = wkv_backward_direct(w, u, k, v, gz)
    for a, b in zip(got[:4], ref):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    assert np.max(np.abs(got[4])) < 1e-20


@pytest.mark.parametrize("seed", [18, 19])
def test_gated_scales_bound_the_gradients(seed):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-3, 1, 3))
    u = rng.normal(0, 0.5, 3)
    k, v, r, gz = (rng.normal(0, 1.5, (2, 9, 3)) for _ in range(4))
    grads, scales = wkv_gated_backward(w, u, k, v, r, gz, return_scale=True)
    for g, s in zip(grads, scales):
        assert np.all(np.abs(g) <= s * (1 + 1e-12) + 1e-300)


@pytest.mark.parametrize("seed", [0, 1])
def test_gated_recurrent_forms_match_direct(seed):
    """The O(T) gated forward and backward (long-sequence references) against the direct sums."""
    rng = np.random.default_rng(seed + 40)
    B, T, C = 2, 37, 5
    w = np.exp(rng.uniform(-3, 1, C))
    u = rng.normal(0, 0.5, C)
    k = rng.normal(0, 1.5, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    r = rng.normal(0, 2, (B, T, C))
    gz = rng.normal(0, 1, (B, T, C))
    z, sz = wkv_gated(w, u, k, v, r, return_scale=True)
    z2, sz2 = wkv_gated_recurrent(w, u, k, v, r, return_scale=True)
    assert np.max(np.abs(z - z2) / sz) <= 1e-12 and np.max(np.abs(sz - sz2) / sz) <= 1e-12
    ref, ref_s = wkv_gated_backward(w, u, k, v, r, gz, return_scale=True)
    got, got_s = wkv_gated_backward_recurrent(w, u, k, v, r, gz, return_scale=True)
    for g, gr, s, gs in zip(got, ref, ref_s, got_s):
        fl = 1e-300 + 2.0 ** -200 * s.max()
        assert np.max(np.abs(g - gr) / np.maximum(s, fl)) <= 1e-12
        assert np.max(np.abs(gs - s) / np.maximum(s, fl)) <= 1e-12
