"""Pins for the float64 oracle: each checks it against something other than itself.

Sources: page "Reinventing RNNs for the Transformer Era: RWKV" (velog review):
section "WKV 연산자" (WKV equation), the AFT equation and the linear decay
w_{t,i} = -(t-i) w of its Background section, section "RNN-유사추론" (RNN-mode
equation) and its list of RNN properties (causality, constant memory).  Page
"Transformers are RNNs" (linear attention review), section on causal masking
and cumulative sums (S_i, Z_i).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (
    EMPTY_P,
    scaled_error,
    state_log_b,
    state_ratio,
    wkv_direct,
    wkv_direct_at,
    wkv_mp,
    wkv_recurrent,
    wkv_step_ref,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "wkv_hand_examples.json")


def rand_inputs(B, T, C, seed, k_std=1.0, w_lo=-3.0, w_hi=1.0, u_std=0.5):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(w_lo, w_hi, C))
    u = rng.normal(0, u_std, C)
    k = rng.normal(0, k_std, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    return w, u, k, v


def _parse_log(s):
    s = s.strip()
    if s == "0":
        return 0.0
    assert s.startswith("ln ")
    return math.log(float(s[3:]))


# --------------------------------------------------------------------------
# Pin: hand-derived worked examples (exact rationals)
# --------------------------------------------------------------------------

def load_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_hand_examples(ex):
    T = len(ex["v"])
    # embed the example lane among other lanes to check that lanes stay independent
    B, C = 2, 3
    w, u, k, v = rand_inputs(B, T, C, seed=7)
    w[1] = _parse_log(ex["w"])
    u[1] = _parse_log(ex["u"])
    k[1, :, 1] = [_parse_log(x) for x in ex["k"]]
    v[1, :, 1] = ex["v"]
    want = np.array([float(Fraction(x)) for x in ex["y"]])
    for y in (wkv_direct(w, u, k, v), wkv_recurrent(w, u, k, v)):
        np.testing.assert_allclose(y[1, :, 1], want, rtol=1e-14, atol=1e-15)
    # the 50-digit evaluation that pins the float64 forms is itself pinned here
    y_mp = wkv_mp(w[1:2], u[1:2], k[1:2, :, 1:2], v[1:2, :, 1:2]).astype(np.float64)
    np.testing.assert_allclose(y_mp[0, :, 0], want, rtol=1e-15, atol=1e-16)
    for t in range(T):
        yt, _ = wkv_direct_at(w[1], u[1], k[1, :, 1], v[1, :, 1], t)
        assert abs(yt - want[t]) <= 1e-14 * max(1.0, abs(want[t]))


def _mutant(w, u, k, v, kind):
    """Plausible wrong readings of the WKV equation, for one lane (1-D k, v)."""
    T = len(k)
    y = np.empty(T)
    for t in range(T):
        num = den = 0.0
        for i in range(t):
            dist = {"decay_t_minus_i": t - i, "no_decay_offset": t - 1 - i}.get(kind, t - 1 - i)
            wt = math.exp(-dist * w + k[i])
            if kind == "bonus_on_past":
                wt *= math.exp(u)
            if kind == "kv_swapped":
                wt = math.exp(-dist * w + v[i])
            num += wt * (k[i] if kind == "kv_swapped" else v[i])
            den += wt
        if kind != "no_current_term" or t == 0:
            cur = math.exp((0.0 if kind == "no_bonus" else u) + (v[t] if kind == "kv_swapped" else k[t]))
            num += cur * (k[t] if kind == "kv_swapped" else v[t])
            den += cur
        y[t] = num / den
    return y


@pytest.mark.parametrize("kind", ["decay_t_minus_i", "bonus_on_past", "kv_swapped", "no_current_term", "no_bonus"])
def test_hand_examples_reject_wrong_readings(kind):
    """Every plausible misreading disagrees with at least one hand example."""
    rejected = False
    for ex in load_examples():
        w = _parse_log(ex["w"])
        u = _parse_log(ex["u"])
        k = np.array([_parse_log(x) for x in ex["k"]])
        v = np.array(ex["v"], dtype=np.float64)
        want = np.array([float(Fraction(x)) for x in ex["y"]])
        if np.max(np.abs(_mutant(w, u, k, v, kind) - want)) > 1e-9:
            rejected = True
    assert rejected, kind


# --------------------------------------------------------------------------
# Pin: high-precision brute force (mpmath, 50 digits)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_direct_and_recurrent_match_mpmath(seed):
    w, u, k, v = rand_inputs(2, 12, 3, seed, k_std=2.0)
    ref = wkv_mp(w, u, k, v).astype(np.float64)
    yd, s = wkv_direct(w, u, k, v, return_scale=True)
    yr = wkv_recurrent(w, u, k, v)
    assert scaled_error(yd, ref, s) < 1e-14
    assert scaled_error(yr, ref, s) < 1e-14


# --------------------------------------------------------------------------
# Pin: the two independent forms agree (WKV equation vs RNN-mode equation)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape,seed,k_std", [((1, 64, 64), 0, 1.0), ((3, 200, 17), 3, 2.0), ((2, 513, 5), 4, 1.0)])
def test_direct_vs_recurrent(shape, seed, k_std):
    w, u, k, v = rand_inputs(*shape, seed, k_std=k_std, w_lo=-6.0)
    yd, sd = wkv_direct(w, u, k, v, return_scale=True)
    yr, sr = wkv_recurrent(w, u, k, v, return_scale=True)
    assert scaled_error(yr, yd, sd) < 1e-12
    np.testing.assert_allclose(sr, sd, rtol=1e-12)


def test_direct_at_matches_direct():
    w, u, k, v = rand_inputs(2, 40, 4, seed=11)
    y, s = wkv_direct(w, u, k, v, return_scale=True)
    for b, c, t in [(0, 0, 0), (1, 3, 39), (0, 2, 17), (1, 1, 1)]:
        yt, st = wkv_direct_at(w[c], u[c], k[b, :, c], v[b, :, c], t)
        assert abs(yt - y[b, t, c]) <= 1e-14 * s[b, t, c]
        assert abs(st - s[b, t, c]) <= 1e-14 * s[b, t, c]


# --------------------------------------------------------------------------
# Pins: closed forms and special cases
# --------------------------------------------------------------------------

def test_single_token_returns_v():
    """T = 1: only the current term exists, so y = v exactly."""
    w, u, k, v = rand_inputs(4, 1, 9, seed=2, k_std=3.0)
    assert np.array_equal(wkv_direct(w, u, k, v), v)
    assert np.array_equal(wkv_recurrent(w, u, k, v), v)


def test_constant_v_gives_constant_y():
    """The weights are normalised: v = c for all t gives y = c."""
    w, u, k, _ = rand_inputs(2, 50, 6, seed=5, k_std=2.0)
    v = np.full(k.shape, -1.75)
    for y in (wkv_direct(w, u, k, v), wkv_recurrent(w, u, k, v)):
        np.testing.assert_allclose(y, -1.75, rtol=1e-14)


def test_convex_bounds_and_scale():
    """y_t is a convex combination of v_1..v_t; s_t >= |y_t|, equal when v > 0."""
    w, u, k, v = rand_inputs(2, 80, 5, seed=6, k_std=2.0)
    y, s = wkv_direct(w, u, k, v, return_scale=True)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)
    assert np.all(s >= np.abs(y) - 1e-12)
    y2, s2 = wkv_direct(w, u, k, np.abs(v) + 0.1, return_scale=True)
    np.testing.assert_allclose(s2, y2, rtol=1e-13)


def test_causality():
    """Changing k, v after time t leaves y_1..y_t unchanged (page's RNN properties: causality)."""
    w, u, k, v = rand_inputs(2, 60, 4, seed=8)
    y = wkv_recurrent(w, u, k, v)
    yd = wkv_direct(w, u, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, 31:] += 5.0
    v2[:, 31:] = -v2[:, 31:]
    assert np.array_equal(wkv_recurrent(w, u, k2, v2)[:, :31], y[:, :31])
    assert np.array_equal(wkv_direct(w, u, k2, v2)[:, :31], yd[:, :31])
    assert not np.allclose(wkv_direct(w, u, k2, v2)[:, 31:], yd[:, 31:])


def _aft_linear_decay(w, u_unused, k, v):
    """AFT attention Attn+(W,K,V)_t with w_{t,i} = -(t-i) w, sum over i <= t (Background section)."""
    B, T, C = k.shape
    y = np.empty_like(k)
    for t in range(T):
        dist = np.arange(t, -1, -1, dtype=np.float64)  # t - i for i = 0..t
        e = k[:, : t + 1, :] - dist[None, :, None] * w[None, None, :]
        e = np.exp(e - e.max(axis=1, keepdims=True))
        y[:, t, :] = (e * v[:, : t + 1, :]).sum(axis=1) / e.sum(axis=1)
    return y


def test_u_equal_w_reduces_to_aft():
    """u = w: dividing num and den by e^{w} turns the WKV weights into AFT's e^{-(t-i)w + k_i}."""
    w, _, k, v = rand_inputs(2, 70, 5, seed=9, k_std=2.0)
    y = wkv_direct(w, w, k, v)
    np.testing.assert_allclose(y, _aft_linear_decay(w, None, k, v), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(wkv_recurrent(w, w, k, v), y, rtol=1e-12, atol=1e-13)


def test_u_equal_w_large_gives_current_v():
    """u = w -> infinity: AFT with infinitely fast decay keeps only the current token."""
    _, _, k, v = rand_inputs(2, 30, 4, seed=10)
    w = np.full(4, 60.0)
    for y in (wkv_direct(w, w, k, v), wkv_recurrent(w, w, k, v)):
        np.testing.assert_allclose(y, v, rtol=0, atol=1e-18 + 1e-20)


def test_large_w_keeps_newest_past_token():
    """w -> infinity with fixed u: only the newest past token (undecayed) and the current one remain."""
    _, u, k, v = rand_inputs(2, 30, 4, seed=12)
    w = np.full(4, 1000.0)
    y = wkv_recurrent(w, u, k, v)
    want = np.empty_like(v)
    want[:, 0] = v[:, 0]
    ep = np.exp(k[:, :-1])
    ec = np.exp(u[None, None, :] + k[:, 1:])
    want[:, 1:] = (ep * v[:, :-1] + ec * v[:, 1:]) / (ep + ec)
    np.testing.assert_allclose(y, want, rtol=1e-13)
    np.testing.assert_allclose(wkv_direct(w, u, k, v), want, rtol=1e-13)
    assert np.max(np.abs(y[:, 1:] - v[:, 1:])) > 0.1  # so y is not v_t here


def test_bonus_limits():
    """u -> +inf gives v_t; u -> -inf gives the past-only weighted mean (t >= 2)."""
    w, _, k, v = rand_inputs(2, 25, 3, seed=13)
    yp = wkv_recurrent(w, np.full(3, 300.0), k, v)
    np.testing.assert_allclose(yp, v, rtol=0, atol=1e-12)
    yn = wkv_recurrent(w, np.full(3, -300.0), k, v)
    with np.errstate(invalid="ignore"):  # t = 1 has no past: 0/0 there, unused
        past = wkv_direct(w, np.full(3, -np.inf), k, v)  # current weight exactly 0 for t >= 2
    np.testing.assert_allclose(yn[:, 1:], past[:, 1:], rtol=1e-12)
    # past-only mean at t=2 is v_1
    np.testing.assert_allclose(yn[:, 1], v[:, 0], rtol=1e-12)


def test_no_decay_is_causal_linear_attention():
    """w = 0: per channel, causal linear attention with feature map e^{k} and query 1.

    Linear-attention page: S_i = sum_{j<=i} phi(K_j) V_j, Z_i = sum_{j<=i} phi(K_j),
    V'_i = phi(Q_i) S_i / phi(Q_i) Z_i.  With u = 0 it is exactly S_t / Z_t; with
    w = u = k = 0 it is the cumulative mean of v.
    """
    _, _, k, v = rand_inputs(2, 90, 4, seed=14)
    zero = np.zeros(4)
    S = np.cumsum(np.exp(k) * v, axis=1)
    Z = np.cumsum(np.exp(k), axis=1)
    np.testing.assert_allclose(wkv_direct(zero, zero, k, v), S / Z, rtol=1e-12)
    np.testing.assert_allclose(wkv_recurrent(zero, zero, k, v), S / Z, rtol=1e-12)
    mean = np.cumsum(v, axis=1) / np.arange(1, 91)[None, :, None]
    np.testing.assert_allclose(wkv_recurrent(zero, zero, np.zeros_like(k), v), mean, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("q", [0.3, 0.9, 0.999])
def test_geometric_decay_closed_form(q):
    """k = u = 0 and one-hot v at s: y_t = q^{t-1-s} / D_t with D_t = 1 + (1-q^{t-1})/(1-q) (1-based t)."""
    T, s = 400, 5  # s is 1-based
    w = np.array([-math.log(q)])
    k = np.zeros((1, T, 1))
    v = np.zeros((1, T, 1))
    v[0, s - 1, 0] = 1.0
    y = wkv_recurrent(w, np.zeros(1), k, v)[0, :, 0]
    for t in range(1, T + 1):
        D = 1.0 + (1.0 - q ** (t - 1)) / (1.0 - q)
        want = 0.0 if t < s else (1.0 / D if t == s else q ** (t - 1 - s) / D)
        assert abs(y[t - 1] - want) <= 1e-13 * max(want, 1e-300) + 1e-300, t


@pytest.mark.parametrize("shift", [200.0, -200.0])
def test_key_shift_and_value_affine_invariance(shift):
    """k -> k + c cancels in the ratio; v -> alpha v + beta maps y -> alpha y + beta."""
    w, u, k, v = rand_inputs(2, 120, 4, seed=15, k_std=2.0)
    y = wkv_recurrent(w, u, k, v)
    np.testing.assert_allclose(wkv_recurrent(w, u, k + shift, v), y, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(wkv_direct(w, u, k + shift, v), y, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(wkv_recurrent(w, u, k, -3.0 * v + 0.5), -3.0 * y + 0.5, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Pins: RNN-mode state (constant-size state lets a sequence resume anywhere)
# --------------------------------------------------------------------------

def test_resume_from_state_matches_full_run():
    w, u, k, v = rand_inputs(3, 100, 6, seed=16, k_std=2.0)
    y_full = wkv_direct(w, u, k, v)
    y1, st = wkv_recurrent(w, u, k[:, :37], v[:, :37], return_state=True)
    y2 = wkv_recurrent(w, u, k[:, 37:], v[:, 37:], state=st)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y_full, rtol=1e-12, atol=1e-13)


def test_step_chain_matches_direct():
    """T successive single steps from the empty state reproduce the WKV equation."""
    w, u, k, v = rand_inputs(2, 45, 5, seed=17, k_std=2.0)
    y_ref, s = wkv_direct(w, u, k, v, return_scale=True)
    a = np.zeros((2, 5))
    b = np.zeros((2, 5))
    p = np.full((2, 5), EMPTY_P)
    ys = []
    for t in range(45):
        yt, (a, b, p) = wkv_step_ref(w, u, k[:, t], v[:, t], a, b, p)
        ys.append(yt)
    assert scaled_error(np.stack(ys, axis=1), y_ref, s) < 1e-12
    # the state equals (A, B) of the definition after T tokens
    dist = np.arange(44, -1, -1, dtype=np.float64)
    logB = np.log(np.sum(np.exp(k - dist[None, :, None] * w[None, None, :]), axis=1))
    np.testing.assert_allclose(state_log_b(a, b, p), logB, rtol=0, atol=1e-12)


def test_state_invariants_are_representation_free():
    """(a e^d, b e^d, p - d) is the same state: log B and A/B do not change."""
    rng = np.random.default_rng(18)
    a, b, p = rng.normal(size=5), rng.uniform(0.5, 3, 5), rng.normal(size=5)
    d = rng.normal(size=5) * 10
    np.testing.assert_allclose(state_log_b(a * np.exp(d), b * np.exp(d), p - d), state_log_b(a, b, p), atol=1e-12)
    np.testing.assert_allclose(state_ratio(a * np.exp(d), b * np.exp(d), p - d), state_ratio(a, b, p), rtol=1e-12)


def test_scaled_error_metric():
    y = np.array([1.0, -2.0, 0.0])
    s = np.array([2.0, 4.0, 0.0])
    assert scaled_error(y, y, s) == 0.0
    assert scaled_error(y + np.array([0.1, 0.0, 0.0]), y, s) == pytest.approx(0.05)
    assert scaled_error(np.array([1.0, -2.0, 1e-30]), y, s) == math.inf
    assert scaled_error(np.array([np.nan, -2.0, 0.0]), y, s) == math.inf
