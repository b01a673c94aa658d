"""Pins of the float64 causal linear attention oracle (no GPU).

Against what the oracle does not compute itself: torch's elu (a library routine), a hand-worked
two-position example, the page's two forms (masked sums and cumulative states) against each
other, the one-dimensional case that is the WKV operator with w = 0 and u = 0 (a different
oracle function), causality, and the invariances of a normalised positive-weight average.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import wkv_direct
from oracle.linear_attention import elu_feature, linear_attention_direct, linear_attention_recurrent

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "linear_attention_hand_example.json")


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(0.0, scale, shape)


def test_feature_map_is_elu_plus_one():
    x = np.linspace(-30, 30, 1201)
    ref = torch.nn.functional.elu(torch.from_numpy(x)).numpy() + 1.0
    # torch forms (e^x - 1) + 1, which rounds by up to 2^-53 absolute where e^x is tiny
    np.testing.assert_allclose(elu_feature(x), ref, rtol=1e-15, atol=2e-16)
    assert np.all(elu_feature(np.array([-700.0, -1.0, 0.0, 2.0])) > 0)


def test_hand_example():
    """Two positions, D = 1, M = 1, worked by hand (tests/golden)."""
    ex = json.load(open(GOLDEN))
    for case in ex["cases"]:
        q = np.array(case["q"], dtype=np.float64)[None, :, None]
        k = np.array(case["k"], dtype=np.float64)[None, :, None]
        v = np.array(case["v"], dtype=np.float64)[None, :, None]
        want = np.array(case["out"], dtype=np.float64)
        for f in (linear_attention_direct, linear_attention_recurrent):
            np.testing.assert_allclose(f(q, k, v, feature=case["feature"])[0, :, 0], want, rtol=1e-14)


@pytest.mark.parametrize("shape", [(2, 9, 4, 3), (1, 30, 8, 8), (3, 5, 1, 6)])
def test_direct_matches_recurrent(shape):
    bh, n, d, m = shape
    q, k, v = rand((bh, n, d), 1), rand((bh, n, d), 2), rand((bh, n, m), 3)
    np.testing.assert_allclose(linear_attention_direct(q, k, v), linear_attention_recurrent(q, k, v),
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("shape", [(2, 9, 4, 3), (1, 40, 8, 8)])
def test_recurrent_scale_matches_direct(shape):
    """The cumulative |v| state gives the direct form's scale; the scale bounds |out| and equals
    |out| when every value has one sign."""
    bh, n, d, m = shape
    q, k, v = rand((bh, n, d), 4), rand((bh, n, d), 5), rand((bh, n, m), 6)
    out_d, sc_d = linear_attention_direct(q, k, v, return_scale=True)
    out_r, sc_r = linear_attention_recurrent(q, k, v, return_scale=True)
    np.testing.assert_allclose(out_r, out_d, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sc_r, sc_d, rtol=1e-12, atol=0)
    assert np.all(np.abs(out_r) <= sc_r * (1 + 1e-12))
    _, sc_pos = linear_attention_recurrent(q, k, np.abs(v), return_scale=True)
    np.testing.assert_allclose(sc_pos, linear_attention_recurrent(q, k, np.abs(v)), rtol=1e-12)


def test_one_dimension_is_wkv_without_decay_or_bonus():
    """D = 1 with phi(k) = e^k and any positive query is sum_{j<=i} e^{k_j} v_j / sum e^{k_j}:
    the WKV equation at w = 0, u = 0, one channel per value column."""
    n, m = 12, 5
    kk = rand((1, n, 1), 4)
    v = rand((1, n, m), 5)
    q = np.abs(rand((1, n, 1), 6)) + 0.1
    out = linear_attention_direct(q, np.exp(kk), v, feature=False)
    w = np.zeros(m)
    u = np.zeros(m)
    ref = wkv_direct(w, u, np.repeat(kk, m, axis=2), v)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_causal():
    q, k, v = rand((2, 10, 3), 7), rand((2, 10, 3), 8), rand((2, 10, 4), 9)
    base = linear_attention_direct(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, 6:] += 3.0
    v2[:, 6:] -= 5.0
    changed = linear_attention_direct(q, k2, v2)
    np.testing.assert_array_equal(changed[:, :6], base[:, :6])
    assert np.all(np.abs(changed[:, 6:] - base[:, 6:]) > 0)


def test_average_invariances():
    """Positive weights normalised to one: outputs are convex combinations of the values,
    affine in v, unchanged when a query's feature vector is scaled, and the first output
    is the first value."""
    q, k, v = rand((2, 11, 4), 10), rand((2, 11, 4), 11), rand((2, 11, 3), 12)
    out, scale = linear_attention_direct(q, k, v, return_scale=True)
    np.testing.assert_allclose(out[:, 0], v[:, 0], rtol=1e-14)
    assert np.all(np.abs(out) <= scale * (1 + 1e-12))
    np.testing.assert_allclose(linear_attention_direct(q, k, 2.5 * v - 1.0), 2.5 * out - 1.0, rtol=1e-12, atol=1e-13)
    fq, fk = elu_feature(q), elu_feature(k)
    np.testing.assert_allclose(linear_attention_direct(3.0 * fq, fk, v, feature=False), out, rtol=1e-13)
    cummax = np.maximum.accumulate(v, axis=1)
    cummin = np.minimum.accumulate(v, axis=1)
    assert np.all(out <= cummax + 1e-12) and np.all(out >= cummin - 1e-12)
