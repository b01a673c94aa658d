"""Float64 gradients of the WKV operator (test infrastructure only).

Only tests and the smoke check use this module; the libwkv library never does.

What it computes
----------------
Page "Reinventing RNNs for the Transformer Era: RWKV" (velog paper review),
section "WKV 연산자", WKV equation: per lane (b, c) and time t,

    y_t = sum_{i<=t} alpha_{t,i} v_i,   alpha_{t,i} = e^{E_{t,i}} / sum_j e^{E_{t,j}},
    E_{t,i} = -(t-1-i) w + k_i  (i < t),   E_{t,t} = u + k_t.

The same page's section "Transformer-유사학습" trains the model in the
time-parallel mode, which needs the gradients of a loss L through WKV.  Given
gy_t = dL/dy_t, differentiating the sums term by term (alpha is a softmax over
i of E_{t,i}, and dy_t/dE_{t,i} = alpha_{t,i} (v_i - y_t)):

    dL/dv_i = sum_{t>=i} gy_t alpha_{t,i}
    dL/dk_i = sum_{t>=i} gy_t alpha_{t,i} (v_i - y_t)
    dL/du   = sum_t gy_t alpha_{t,t} (v_t - y_t)
    dL/dw   = sum_t gy_t sum_{i<t} -(t-1-i) alpha_{t,i} (v_i - y_t)

w and u are per channel; ``wkv_backward_direct`` returns their gradients per
lane, shape [B, C] (the channel gradient is the sum over the batch).  Arithmetic
is float64 with the same exact max-shift as ``wkv_direct``; O(T^2) per lane.
"""
from __future__ import annotations

import numpy as np

from .wkv_oracle import _channel_vectors, _f64


def wkv_backward_direct(w, u, k, v, gy, return_scale=False):
    """Gradients of sum(gy * y) with respect to w, u (per lane), k and v.

    k, v, gy: [B, T, C]; w, u: [C].  Returns (gw [B, C], gu [B, C], gk, gv).
    With ``return_scale`` also returns the scales the same sums take with every
    term replaced by its magnitude (|gy|, and |v_i| + |y_t| for v_i - y_t): the
    denominators of the scale-normalised gradient error.
    """
    k = _f64(k)
    v = _f64(v)
    gy = _f64(gy)
    nb, T, C = k.shape
    w, u = _channel_vectors(w, u, C)
    gk = np.zeros((nb, T, C))
    gv = np.zeros((nb, T, C))
    gw = np.zeros((nb, C))
    gu = np.zeros((nb, C))
    sk = np.zeros((nb, T, C))
    sv = np.zeros((nb, T, C))
    sw = np.zeros((nb, C))
    su = np.zeros((nb, C))
    for t in range(T):
        dist = np.arange(t - 1, -1, -1, dtype=np.float64)  # t-1-i for i = 0..t-1
        e_all = np.concatenate([k[:, :t, :] - dist[None, :, None] * w[None, None, :],
                                (u[None, :] + k[:, t, :])[:, None, :]], axis=1)
        vals = v[:, : t + 1, :]
        e = np.exp(e_all - e_all.max(axis=1, keepdims=True))
        alpha = e / e.sum(axis=1, keepdims=True)  # [B, t+1, C]
        yt = (alpha * vals).sum(axis=1)  # [B, C]
        g = gy[:, t, :]
        ga = g[:, None, :] * alpha
        diff = vals - yt[:, None, :]
        gv[:, : t + 1, :] += ga
        gk[:, : t + 1, :] += ga * diff
        gu += ga[:, t, :] * diff[:, t, :]
        gw -= (dist[None, :, None] * ga[:, :t, :] * diff[:, :t, :]).sum(axis=1)
        if return_scale:
            aa = np.abs(g)[:, None, :] * alpha
            mag = np.abs(vals) + np.abs(yt)[:, None, :]
            sv[:, : t + 1, :] += aa
            sk[:, : t + 1, :] += aa * mag
            su += aa[:, t, :] * mag[:, t, :]
            sw += (dist[None, :, None] * aa[:, :t, :] * mag[:, :t, :]).sum(axis=1)
    if return_scale:
        return (gw, gu, gk, gv), (sw, su, sk, sv)
    return gw, gu, gk, gv


def wkv_backward_recurrent(w, u, k, v, gy, return_scale=False):
    """The same gradients as ``wkv_backward_direct`` in O(T) per lane: a forward pass for
    the outputs and denominators, then one reverse pass over time.

    With D_t = B_t + e^{u+k_t} the WKV denominator of output t (B_t the RNN-mode state of
    section "RNN-유사추론") and q_t = gy_t / D_t, the sums over later outputs

        G_i  = sum_{t>i} q_t e^{-(t-1-i) w},          H_i  = sum_{t>i} q_t y_t e^{-(t-1-i) w},
        G'_i = sum_{t>i} (t-1-i) q_t e^{-(t-1-i) w},  H'_i = the same with q_t y_t,

    obey G_{i-1} = q_i + e^{-w} G_i (H alike) and G'_{i-1} = e^{-w} (G'_i + G_i) (H' alike),
    and the derivatives of the WKV equation are

        dL/dv_i = e^{k_i} G_i + e^{u+k_i} q_i
        dL/dk_i = e^{k_i} (v_i G_i - H_i) + e^{u+k_i} q_i (v_i - y_i)
        dL/du   = sum_i e^{u+k_i} q_i (v_i - y_i)
        dL/dw   = -sum_i e^{k_i} (v_i G'_i - H'_i).

    The reverse sums are kept as coefficient times e^{gamma}, gamma the largest exponent
    -(t-1-i) w - log D_t among their terms (so e^{k_i + gamma} <= 1: D_t contains the term
    of token i).  With ``return_scale`` the same sums are formed with |gy| and magnitudes
    (|v_i| + |y_t| for v_i - y_t): the scales ``wkv_backward_direct`` returns.
    """
    k = _f64(k)
    v = _f64(v)
    gy = _f64(gy)
    nb, T, C = k.shape
    w, u = _channel_vectors(w, u, C)
    # forward: outputs y_t and log D_t, RNN-mode state (a, b, p) with B = b e^p
    y = np.empty((nb, T, C))
    logd = np.empty((nb, T, C))
    a = np.zeros((nb, C))
    b = np.zeros((nb, C))
    p = np.full((nb, C), -np.inf)
    for t in range(T):
        uk = u + k[:, t, :]
        q = np.maximum(p, uk)
        e_state = np.exp(p - q)
        e_cur = np.exp(uk - q)
        den = e_state * b + e_cur
        y[:, t, :] = (e_state * a + e_cur * v[:, t, :]) / den
        logd[:, t, :] = q + np.log(den)
        pw = p - w
        q2 = np.maximum(pw, k[:, t, :])
        f_old = np.exp(pw - q2)
        f_new = np.exp(k[:, t, :] - q2)
        a = f_old * a + f_new * v[:, t, :]
        b = f_old * b + f_new
        p = q2
    # reverse: (G, H, G', H') and their magnitude twins share the reference gamma
    z = lambda: np.zeros((nb, C))  # noqa: E731
    g, h, g1, h1 = z(), z(), z(), z()
    ga, ha, g1a, h1a = z(), z(), z(), z()
    gamma = np.full((nb, C), -np.inf)
    gk = np.empty((nb, T, C))
    gv = np.empty((nb, T, C))
    gw = z()
    gu = z()
    sk = np.empty((nb, T, C))
    sv = np.empty((nb, T, C))
    sw = z()
    su = z()
    for i in range(T - 1, -1, -1):
        ki, vi, yi, gi = k[:, i, :], v[:, i, :], y[:, i, :], gy[:, i, :]
        # the sums over t > i are complete here
        with np.errstate(invalid="ignore"):
            ek = np.where(np.isneginf(gamma), 0.0, np.exp(ki + gamma))
        cur = np.exp(u + ki - logd[:, i, :])  # e^{u+k_i} / D_i
        gv[:, i, :] = ek * g + cur * gi
        gk[:, i, :] = ek * (vi * g - h) + cur * gi * (vi - yi)
        gu += cur * gi * (vi - yi)
        gw -= ek * (vi * g1 - h1)
        if return_scale:
            mag = np.abs(vi) + np.abs(yi)
            sv[:, i, :] = ek * ga + cur * np.abs(gi)
            sk[:, i, :] = ek * (np.abs(vi) * ga + ha) + cur * np.abs(gi) * mag
            su += cur * np.abs(gi) * mag
            sw += ek * (np.abs(vi) * g1a + h1a)
        # extend the sums to t > i - 1: decay the old terms by e^{-w}, add q_i
        new = -logd[:, i, :]
        gnext = np.maximum(gamma - w, new)
        f_old = np.exp(gamma - w - gnext)
        f_new = np.exp(new - gnext)
        g1 = f_old * (g1 + g)
        h1 = f_old * (h1 + h)
        g = f_old * g + f_new * gi
        h = f_old * h + f_new * gi * yi
        if return_scale:
            g1a = f_old * (g1a + ga)
            h1a = f_old * (h1a + ha)
            ga = f_old * ga + f_new * np.abs(gi)
            ha = f_old * ha + f_new * np.abs(gi) * np.abs(yi)
        gamma = gnext
    if return_scale:
        return (gw, gu, gk, gv), (sw, su, sk, sv)
    return gw, gu, gk, gv
