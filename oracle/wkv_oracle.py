"""Plain float64 evaluation of the RWKV-4 WKV operator (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this module;
the libwkv library never does.

What it computes
----------------
Page "Reinventing RNNs for the Transformer Era: RWKV" (velog paper review),
section "WKV 연산자" (the WKV operator), WKV equation.  For every batch b,
channel c and time t = 1..T:

    wkv_t = ( sum_{i=1}^{t-1} exp(-(t-1-i) w + k_i) v_i  +  exp(u + k_t) v_t )
            / ( sum_{i=1}^{t-1} exp(-(t-1-i) w + k_i)     +  exp(u + k_t) )

w and u are per-channel vectors: the same section calls the decay channel-wise,
and the RNN-mode section ("RNN-유사추론") lists w as the per-channel decay rate
and u as the constant vector that corrects the current token's weight.  Every
(b, c) lane is independent because the products are elementwise.

The RNN-mode section writes WKV_t = (A_t + e^{u+k_t} v_t) / (B_t + e^{u+k_t})
with (A_t, B_t) the per-channel hidden state but never writes how the state
advances.  The reading used here is the one that reproduces the WKV equation:

    A_1 = B_1 = 0,   A_{t+1} = e^{-w} A_t + e^{k_t} v_t,   B_{t+1} = e^{-w} B_t + e^{k_t}

(the newest past token carries no decay).  A state triple (a, b, p) stands for
A = a e^p, B = b e^p; the empty state is a = b = 0 with p = EMPTY_P.

Arithmetic is float64 throughout.  Rescaling by a maximum exponent is an exact
identity (it multiplies numerator and denominator by the same factor) and is
used only so that shifted inputs (k + 200) do not overflow float64.
"""
from __future__ import annotations

import numpy as np

#: p of the empty state (a = b = 0): a finite stand-in for minus infinity.
EMPTY_P = -1.0e38


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _channel_vectors(w, u, C):
    w = _f64(w).reshape(-1)
    u = _f64(u).reshape(-1)
    if w.shape != (C,) or u.shape != (C,):
        raise ValueError(f"w and u must have {C} entries, got {w.shape} and {u.shape}")
    return w, u


def wkv_direct(w, u, k, v, return_scale=False):
    """The WKV equation evaluated term by term, O(T^2) per lane.

    k, v: [B, T, C]; w, u: [C].  Returns y [B, T, C] (and the scale s, the same
    convex weights applied to |v|, when ``return_scale``).

    Time index: Python's 0-based t is the page's t+1; the decay of past token i
    at output t is (t-1-i) in either indexing because both shift by one.
    """
    k = _f64(k)
    v = _f64(v)
    nb, T, C = k.shape
    w, u = _channel_vectors(w, u, C)
    y = np.empty((nb, T, C))
    s = np.empty((nb, T, C))
    for t in range(T):
        # past tokens i = 0..t-1 carry exponent -(t-1-i) w + k_i
        dist = np.arange(t - 1, -1, -1, dtype=np.float64)
        e_past = k[:, :t, :] - dist[None, :, None] * w[None, None, :]
        # the current token carries u + k_t
        e_cur = (u[None, :] + k[:, t, :])[:, None, :]
        e_all = np.concatenate([e_past, e_cur], axis=1)
        vals = v[:, : t + 1, :]
        m = e_all.max(axis=1, keepdims=True)
        wt = np.exp(e_all - m)
        den = wt.sum(axis=1)
        y[:, t, :] = (wt * vals).sum(axis=1) / den
        s[:, t, :] = (wt * np.abs(vals)).sum(axis=1) / den
    return (y, s) if return_scale else y


def wkv_direct_at(w_c, u_c, k_lane, v_lane, t):
    """The WKV equation for one lane at one 0-based time t, O(t).

    k_lane, v_lane: 1-D arrays over time for a single (b, c); w_c, u_c scalars.
    Returns (y_t, s_t).
    """
    k_lane = _f64(k_lane)
    v_lane = _f64(v_lane)
    w_c = float(w_c)
    u_c = float(u_c)
    dist = np.arange(t - 1, -1, -1, dtype=np.float64)
    e_all = np.concatenate([k_lane[:t] - dist * w_c, [u_c + k_lane[t]]])
    vals = v_lane[: t + 1]
    wt = np.exp(e_all - e_all.max())
    den = wt.sum()
    return float((wt * vals).sum() / den), float((wt * np.abs(vals)).sum() / den)


def wkv_recurrent(w, u, k, v, state=None, return_scale=False, return_state=False):
    """RNN-mode evaluation, O(T): WKV_t = (A_t + e^{u+k_t} v_t) / (B_t + e^{u+k_t}).

    The state is kept as (a, b, p) with A = a e^p, B = b e^p, p the running
    largest exponent; every update multiplies numerator and denominator terms
    by the same e^{-q}, which changes nothing mathematically.

    state: optional (a, b, p) arrays of shape [B, C] to start from (the empty
    state by default).  A fourth array, the |v| accumulator for the scale, may
    be appended; without it the scale of a resumed run counts only new tokens.
    Returns y, plus s (``return_scale``) and the final (a, b, p) (``return_state``).
    """
    nb, T, C = np.shape(k)
    w, u = _channel_vectors(w, u, C)
    if state is None:
        a = np.zeros((nb, C))
        b = np.zeros((nb, C))
        p = np.full((nb, C), -np.inf)
        aabs = np.zeros((nb, C))
    else:
        a, b, p = (_f64(x).reshape(nb, C).copy() for x in state[:3])
        aabs = _f64(state[3]).reshape(nb, C).copy() if len(state) > 3 else np.zeros((nb, C))
    y = np.empty((nb, T, C))
    s = np.empty((nb, T, C)) if return_scale else None
    for t in range(T):
        kt = _f64(k[:, t, :])
        vt = _f64(v[:, t, :])
        # output: past state plus the current token weighted by e^{u+k_t}
        uk = u + kt
        q = np.maximum(p, uk)
        e_state = np.exp(p - q)
        e_cur = np.exp(uk - q)
        den = e_state * b + e_cur
        y[:, t, :] = (e_state * a + e_cur * vt) / den
        if return_scale:
            s[:, t, :] = (e_state * aabs + e_cur * np.abs(vt)) / den
        # state update: decay the past by e^{-w}, add e^{k_t} (v_t, 1)
        pw = p - w
        q2 = np.maximum(pw, kt)
        f_old = np.exp(pw - q2)
        f_new = np.exp(kt - q2)
        a = f_old * a + f_new * vt
        b = f_old * b + f_new
        aabs = f_old * aabs + f_new * np.abs(vt)
        p = q2
    out = [y]
    if return_scale:
        out.append(s)
    if return_state:
        out.append((a, b, p))
    return out[0] if len(out) == 1 else tuple(out)


def wkv_step_ref(w, u, k, v, a, b, p):
    """One RNN-mode step for a batch of independent lanes (decode step).

    k, v, a, b, p: arrays of one common shape (e.g. [N, G, C]); w, u broadcast
    against it (e.g. [G, C]).  The incoming state is A = a e^p, B = b e^p.
    Returns y and the next state (a', b', p') with p' = max(p - w, k).
    """
    w = _f64(w)
    u = _f64(u)
    k = _f64(k)
    v = _f64(v)
    a = _f64(a)
    b = _f64(b)
    p = _f64(p)
    uk = u + k
    q = np.maximum(p, uk)
    e_state = np.exp(p - q)
    e_cur = np.exp(uk - q)
    y = (e_state * a + e_cur * v) / (e_state * b + e_cur)
    pw = p - w
    q2 = np.maximum(pw, k)
    f_old = np.exp(pw - q2)
    f_new = np.exp(k - q2)
    return y, (f_old * a + f_new * v, f_old * b + f_new, q2)


def state_log_b(a, b, p):
    """log B of a state triple: the representation-independent magnitude."""
    return _f64(p) + np.log(_f64(b))


def state_ratio(a, b, p):
    """A / B of a state triple: the representation-independent weighted mean."""
    return _f64(a) / _f64(b)


def scaled_error(y_hat, y_ref, s_ref):
    """max |y_hat - y_ref| / s over all elements (the parity gate).

    s is the same convex combination applied to |v|, so s >= |y| and the
    metric equals plain relative error wherever v has one sign in the window.
    Where s == 0 (all v zero) the result must be exactly 0.  NaN counts as inf.
    """
    y_hat = _f64(y_hat)
    y_ref = _f64(y_ref)
    s_ref = _f64(s_ref)
    err = np.abs(y_hat - y_ref)
    zero = s_ref == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(zero, np.where(err == 0, 0.0, np.inf), err / np.where(zero, 1.0, s_ref))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    return float(ratio.max()) if ratio.size else 0.0
