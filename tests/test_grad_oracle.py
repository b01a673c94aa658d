"""Pins of the float64 WKV gradient oracle (no GPU).

wkv_backward_direct differentiates the WKV equation's sums term by term.  It is
pinned here against things it does not compute itself: central finite
differences of the forward oracle, closed forms (T = 1, constant v), a
conservation law (with gy = 1 the value gradients of a lane sum to T), the
key-shift invariance of the forward, and linearity in gy.

wkv_backward_recurrent reaches the same gradients through a reverse recurrence
over time (O(T), for the long workloads).  It is pinned to the direct sums on
ordinary and ill-conditioned inputs, and to central finite differences itself.
"""
import numpy as np
import pytest

from oracle import wkv_backward_direct, wkv_backward_recurrent, wkv_direct


def rand_inputs(B, T, C, seed, k_std=1.0):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-3.0, 1.0, C))
    u = rng.normal(0.0, 0.5, C)
    k = rng.normal(0.0, k_std, (B, T, C))
    v = rng.normal(0.0, 1.0, (B, T, C))
    gy = rng.normal(0.0, 1.0, (B, T, C))
    return w, u, k, v, gy


def loss(w, u, k, v, gy):
    return float((wkv_direct(w, u, k, v) * gy).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_central_differences(seed):
    """Every partial derivative against (L(x+h) - L(x-h)) / 2h of the forward oracle."""
    B, T, C = 2, 6, 3
    w, u, k, v, gy = rand_inputs(B, T, C, seed, k_std=1.5)
    gw, gu, gk, gv = wkv_backward_direct(w, u, k, v, gy)
    h = 1e-6

    def fd(name, idx):
        args = {"w": w.copy(), "u": u.copy(), "k": k.copy(), "v": v.copy()}
        args[name][idx] += h
        lp = loss(args["w"], args["u"], args["k"], args["v"], gy)
        args[name][idx] -= 2 * h
        lm = loss(args["w"], args["u"], args["k"], args["v"], gy)
        return (lp - lm) / (2 * h)

    for idx in np.ndindex(B, T, C):
        assert abs(fd("k", idx) - gk[idx]) < 1e-7, ("k", idx)
        assert abs(fd("v", idx) - gv[idx]) < 1e-7, ("v", idx)
    for c in range(C):
        # w and u are shared by the batch: their gradient is the sum of the per-lane ones
        assert abs(fd("w", c) - gw[:, c].sum()) < 1e-7, ("w", c)
        assert abs(fd("u", c) - gu[:, c].sum()) < 1e-7, ("u", c)


def test_single_token():
    """T = 1: y = v, so dL/dv = gy and nothing else moves y."""
    w, u, k, v, gy = rand_inputs(3, 1, 5, 7)
    gw, gu, gk, gv = wkv_backward_direct(w, u, k, v, gy)
    np.testing.assert_array_equal(gv, gy)
    assert np.all(gk == 0) and np.all(gu == 0) and np.all(gw == 0)


def test_constant_values():
    """v = c everywhere: y = c whatever the weights, so k, u, w have zero gradient."""
    w, u, k, v, gy = rand_inputs(2, 9, 4, 3, k_std=2.0)
    v[:] = 0.75
    gw, gu, gk, gv = wkv_backward_direct(w, u, k, v, gy)
    assert np.max(np.abs(gk)) < 1e-14 and np.max(np.abs(gu)) < 1e-14 and np.max(np.abs(gw)) < 1e-13


def test_value_gradients_sum_to_t():
    """With gy = 1, sum_i dL/dv_i = sum_t sum_i alpha_{t,i} = T (weights sum to one)."""
    w, u, k, v, _ = rand_inputs(2, 11, 3, 4, k_std=2.0)
    _, _, _, gv = wkv_backward_direct(w, u, k, v, np.ones_like(v))
    np.testing.assert_allclose(gv.sum(axis=1), 11.0, rtol=1e-13)


@pytest.mark.parametrize("shift", [150.0, -150.0])
def test_key_shift_invariance(shift):
    """y does not change when k moves by a constant, so neither do the gradients."""
    w, u, k, v, gy = rand_inputs(2, 10, 3, 5)
    ref = wkv_backward_direct(w, u, k, v, gy)
    got = wkv_backward_direct(w, u, k + shift, v, gy)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_linear_in_upstream_gradient():
    w, u, k, v, gy = rand_inputs(2, 8, 3, 6)
    g1 = wkv_backward_direct(w, u, k, v, gy)
    g2 = wkv_backward_direct(w, u, k, v, -2.5 * gy)
    for a, b in zip(g2, g1):
        np.testing.assert_allclose(a, -2.5 * b, rtol=1e-12, atol=1e-14)


def test_scales_bound_the_gradients():
    w, u, k, v, gy = rand_inputs(2, 12, 3, 8, k_std=2.0)
    grads, scales = wkv_backward_direct(w, u, k, v, gy, return_scale=True)
    for g, s in zip(grads, scales):
        assert np.all(np.abs(g) <= s * (1 + 1e-12) + 1e-300)


def scaled_gap(a, b, s):
    a, b, s = (np.asarray(x, dtype=np.float64) for x in (a, b, s))
    if s.size == 0:
        return 0.0
    floor = 1e-300 + 2.0 ** -200 * s.max()
    return float(np.max(np.abs(a - b) / np.maximum(s, floor)))


def ill_conditioned(case, B=2, T=40, C=6, seed=11):
    w, u, k, v, gy = rand_inputs(B, T, C, seed, k_std=1.5)
    if case == "negative_w":
        w[::2] = -0.05
    elif case == "huge_k_range":
        k[:, ::7, ::2] = 90.0
        k[:, 3::11, 1::3] = -90.0
    elif case == "huge_u":
        u[::2] = 70.0
    elif case == "tiny_u":
        u[::2] = -70.0
    elif case == "w_zero":
        w[:] = 0.0
    elif case == "k_plus_200":
        k += 200.0
    elif case == "k_minus_200":
        k -= 200.0
    elif case == "sparse_gy":
        gy[:, ::3, :] = 0.0
        gy[:, :, ::2] = 0.0
    elif case == "huge_w":
        w[::2] = 1000.0
    return w, u, k, v, gy


@pytest.mark.parametrize("B,T,C,k_std,seed", [(1, 1, 4, 1.0, 0), (2, 2, 3, 1.0, 1), (2, 9, 5, 2.0, 2),
                                               (1, 257, 7, 2.0, 3), (3, 64, 4, 1.0, 4)])
def test_recurrent_matches_direct(B, T, C, k_std, seed):
    """The O(T) reverse recurrence against the term-by-term sums, gradients and scales."""
    w, u, k, v, gy = rand_inputs(B, T, C, seed, k_std=k_std)
    ref, ref_s = wkv_backward_direct(w, u, k, v, gy, return_scale=True)
    got, got_s = wkv_backward_recurrent(w, u, k, v, gy, return_scale=True)
    for name, g, r, s, gs in zip("wukv", got, ref, ref_s, got_s):
        assert scaled_gap(g, r, s) <= 1e-12, name
        assert scaled_gap(gs, s, s) <= 1e-12, name


@pytest.mark.parametrize("case", ["negative_w", "huge_k_range", "huge_u", "tiny_u", "w_zero", "k_plus_200",
                                  "k_minus_200", "sparse_gy", "huge_w"])
def test_recurrent_matches_direct_ill_conditioned(case):
    """Exponent ranges that overflow a plain float64 evaluation: both forms rescale exactly."""
    w, u, k, v, gy = ill_conditioned(case)
    ref, ref_s = wkv_backward_direct(w, u, k, v, gy, return_scale=True)
    got, got_s = wkv_backward_recurrent(w, u, k, v, gy, return_scale=True)
    for name, g, r, s, gs in zip("wukv", got, ref, ref_s, got_s):
        assert np.all(np.isfinite(g)), (case, name)
        assert scaled_gap(g, r, s) <= 1e-12, (case, name)
        assert scaled_gap(gs, s, s) <= 1e-12, (case, name)


@pytest.mark.parametrize("seed", [0, 1])
def test_recurrent_matches_central_differences(seed):
    """The reverse recurrence against (L(x+h) - L(x-h)) / 2h of the forward's defining sums."""
    B, T, C = 2, 7, 3
    w, u, k, v, gy = rand_inputs(B, T, C, seed + 20, k_std=1.5)
    gw, gu, gk, gv = wkv_backward_recurrent(w, u, k, v, gy)
    h = 1e-6

    def fd(name, idx):
        args = {"w": w.copy(), "u": u.copy(), "k": k.copy(), "v": v.copy()}
        args[name][idx] += h
        lp = loss(args["w"], args["u"], args["k"], args["v"], gy)
        args[name][idx] -= 2 * h
        lm = loss(args["w"], args["u"], args["k"], args["v"], gy)
        return (lp - lm) / (2 * h)

    for idx in np.ndindex(B, T, C):
        assert abs(fd("k", idx) - gk[idx]) < 1e-7, ("k", idx)
        assert abs(fd("v", idx) - gv[idx]) < 1e-7, ("v", idx)
    for c in range(C):
        assert abs(fd("w", c) - gw[:, c].sum()) < 1e-7, ("w", c)
        assert abs(fd("u", c) - gu[:, c].sum()) < 1e-7, ("u", c)


def test_recurrent_closed_forms():
    """T = 1 (dL/dv = gy, nothing else) and constant v (no key, bonus or decay gradient)."""
    w, u, k, v, gy = rand_inputs(3, 1, 5, 7)
    gw, gu, gk, gv = wkv_backward_recurrent(w, u, k, v, gy)
    np.testing.assert_array_equal(gv, gy)
    assert np.all(gk == 0) and np.all(gu == 0) and np.all(gw == 0)
    w, u, k, v, gy = rand_inputs(2, 30, 4, 3, k_std=2.0)
    v[:] = -1.25
    gw, gu, gk, gv = wkv_backward_recurrent(w, u, k, v, gy)
    assert np.max(np.abs(gk)) < 1e-13 and np.max(np.abs(gu)) < 1e-13 and np.max(np.abs(gw)) < 1e-12
    _, _, _, gv = wkv_backward_recurrent(w, u, k, v, np.ones_like(v))
    np.testing.assert_allclose(gv.sum(axis=1), 30.0, rtol=1e-13)
