"""Float64 token shift and output gate around WKV (test infrastructure only).

Only tests and the smoke check use this module; the libwkv library never does.

What it computes
----------------
Page "Reinventing RNNs for the Transformer Era: RWKV" (velog paper review):

* Section "토큰 변환" (token shift): the time-mixing block forms its R, K, V inputs (and
  the channel-mixing block its R', K') by linear interpolation between the current and
  the previous time step.  Reading used: for a mix coefficient mu (per channel),
      x^mu_t = mu * x_t + (1 - mu) * x_{t-1},
  with x_{-1} = the token before the sequence (zero for a fresh sequence, or the last
  token of the previous call when a sequence continues).  The projections W_r, W_k, W_v
  that follow are dense products outside this operator.
* Section "출력 게이팅" (output gating): o_t = W_o (sigma(r_t) * wkv_t) with sigma the
  logistic sigmoid; the gated value z_t = sigma(r_t) * wkv_t is what precedes the W_o
  product (which stays outside).

Gradients (for the training mode of section "Transformer-유사학습"), by the chain rule:
  z = s * y with s = sigma(r):  dL/dy = gz * s,  dL/dr = gz * y * s * (1 - s);
  token shift: dL/dx_t = sum_m mu_m g_{m,t} + (1 - mu_m) g_{m,t+1} (g_{m,T} = 0),
               dL/dmu_m = sum_t g_{m,t} (x_t - x_{t-1}),  dL/dx_{-1} = sum_m (1 - mu_m) g_{m,0}.
"""
from __future__ import annotations

import numpy as np

from .wkv_oracle import _f64, wkv_direct, wkv_recurrent
from .wkv_grad import wkv_backward_direct, wkv_backward_recurrent


def sigmoid(r):
    """Logistic sigmoid 1 / (1 + e^{-r}) in float64, without overflow for large |r|."""
    r = _f64(r)
    out = np.empty_like(r)
    pos = r >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-r[pos]))
    e = np.exp(r[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def token_shift(x, mu, x_prev=None):
    """x: [B, T, C]; mu: [M, C]; x_prev: [B, C] or None (zeros).  Returns [M, B, T, C]."""
    x = _f64(x)
    mu = _f64(mu)
    B, T, C = x.shape
    prev = np.zeros((B, 1, C)) if x_prev is None else _f64(x_prev).reshape(B, 1, C)
    shifted = np.concatenate([prev, x[:, :-1, :]], axis=1)  # x_{t-1}
    return mu[:, None, None, :] * x[None] + (1.0 - mu[:, None, None, :]) * shifted[None]


def token_shift_backward(x, mu, g, x_prev=None):
    """Gradients of sum(g * token_shift(x, mu, x_prev)): (gx [B,T,C], gmu [M,B,C] per lane, gprev [B,C])."""
    x = _f64(x)
    mu = _f64(mu)
    g = _f64(g)
    B, T, C = x.shape
    prev = np.zeros((B, 1, C)) if x_prev is None else _f64(x_prev).reshape(B, 1, C)
    shifted = np.concatenate([prev, x[:, :-1, :]], axis=1)
    gx = (mu[:, None, None, :] * g).sum(axis=0)
    gx[:, :-1, :] += ((1.0 - mu[:, None, None, :]) * g[:, :, 1:, :]).sum(axis=0)
    gmu = (g * (x[None] - shifted[None])).sum(axis=2)
    gprev = ((1.0 - mu[:, None, :]) * g[:, :, 0, :]).sum(axis=0)
    return gx, gmu, gprev


def wkv_gated(w, u, k, v, r, return_scale=False):
    """z = sigmoid(r) * WKV(w, u, k, v); with return_scale also the scale s * s_wkv."""
    s = sigmoid(r)
    if return_scale:
        y, sy = wkv_direct(w, u, k, v, return_scale=True)
        return s * y, s * sy
    return s * wkv_direct(w, u, k, v)


def wkv_gated_backward(w, u, k, v, r, gz, return_scale=False):
    """Gradients of sum(gz * sigmoid(r) * WKV): (gw, gu, gk, gv, gr) (+ scales).

    gw, gu per lane [B, C] as in wkv_backward_direct; gr [B, T, C].  The scale of gr is
    |gz| s (1 - s) times the forward's scale of y.
    """
    s = sigmoid(r)
    gz = _f64(gz)
    gy = gz * s
    y, sy = wkv_direct(w, u, k, v, return_scale=True)
    gr = gz * y * s * (1.0 - s)
    if return_scale:
        grads, scales = wkv_backward_direct(w, u, k, v, gy, return_scale=True)
        return (*grads, gr), (*scales, np.abs(gz) * sy * s * (1.0 - s))
    return (*wkv_backward_direct(w, u, k, v, gy), gr)


def wkv_gated_recurrent(w, u, k, v, r, return_scale=False):
    """``wkv_gated`` with the WKV output from the O(T) RNN-mode form (long sequences)."""
    s = sigmoid(r)
    if return_scale:
        y, sy = wkv_recurrent(w, u, k, v, return_scale=True)
        return s * y, s * sy
    return s * wkv_recurrent(w, u, k, v)


def wkv_gated_backward_recurrent(w, u, k, v, r, gz, return_scale=False):
    """``wkv_gated_backward`` from the O(T) forward and reverse recurrences (long sequences)."""
    s = sigmoid(r)
    gz = _f64(gz)
    y, sy = wkv_recurrent(w, u, k, v, return_scale=True)
    gr = gz * y * s * (1.0 - s)
    if return_scale:
        grads, scales = wkv_backward_recurrent(w, u, k, v, gz * s, return_scale=True)
        return (*grads, gr), (*scales, np.abs(gz) * sy * s * (1.0 - s))
    return (*wkv_backward_recurrent(w, u, k, v, gz * s), gr)
