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
