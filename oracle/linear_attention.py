"""Float64 causal linear attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU leg use this module; the libwkv
library never does.

What it computes
----------------
Page "Transformers are RNNs: 선형 어텐션으로 만드는 빠른 자기회귀 트랜스포머" (the linear
transformer review), sections "선형 어텐션과 결합법칙", "특징 맵 선택과 계산 비용" and
"인과 마스킹과 누적합".  For queries Q_i, keys K_j (dimension D) and values V_j (dimension
M) of one sequence (one batch-head), with the feature map phi(x) = elu(x) + 1 applied
elementwise, the causally masked attention is

    V'_i = sum_{j<=i} phi(Q_i)^T phi(K_j) V_j / sum_{j<=i} phi(Q_i)^T phi(K_j).

The same page rewrites it with the cumulative states S_i = sum_{j<=i} phi(K_j) V_j^T and
Z_i = sum_{j<=i} phi(K_j) as V'_i = phi(Q_i)^T S_i / (phi(Q_i)^T Z_i) (the RNN form).

* ``elu_feature``           -- phi(x) = elu(x) + 1 = x + 1 for x > 0, e^x otherwise
* ``linear_attention_direct``    -- the masked sums above, O(N^2) per sequence
* ``linear_attention_recurrent`` -- the cumulative-state form, O(N) per sequence
Both take feature=False to use q, k as given (already mapped, all positive).
"""
from __future__ import annotations

import numpy as np

from .wkv_oracle import _f64


def elu_feature(x):
    """elu(x) + 1: x + 1 for x > 0 and e^x for x <= 0 (so always positive)."""
    x = _f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_attention_direct(q, k, v, feature=True, return_scale=False):
    """q, k: [BH, N, D]; v: [BH, N, M].  Returns out [BH, N, M] (and the scale).

    The scale is the same normalised sum applied to |v| (it bounds |out| and is the
    denominator of the parity metric)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    fq = elu_feature(q) if feature else q
    fk = elu_feature(k) if feature else k
    n = q.shape[1]
    sim = np.einsum("bid,bjd->bij", fq, fk)
    sim = sim * np.tril(np.ones((n, n)))[None]  # j <= i
    den = sim.sum(axis=2, keepdims=True)
    out = (sim @ v) / den
    if return_scale:
        return out, (sim @ np.abs(v)) / den
    return out


def linear_attention_recurrent(q, k, v, feature=True, return_scale=False):
    """The same outputs from the states S_i (D x M) and Z_i (D), one step per position.

    With ``return_scale`` a third state, the same cumulative sum of phi(K_j) |V_j|^T, gives
    the scale (the normalised sum applied to |v|, as ``linear_attention_direct`` returns it)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    fq = elu_feature(q) if feature else q
    fk = elu_feature(k) if feature else k
    bh, n, d = q.shape
    m = v.shape[2]
    s = np.zeros((bh, d, m))
    s_abs = np.zeros((bh, d, m)) if return_scale else None
    z = np.zeros((bh, d))
    out = np.empty((bh, n, m))
    scale = np.empty((bh, n, m)) if return_scale else None
    for i in range(n):
        s += fk[:, i, :, None] * v[:, i, None, :]
        z += fk[:, i, :]
        den = np.einsum("bd,bd->b", fq[:, i, :], z)[:, None]
        out[:, i, :] = np.einsum("bd,bdm->bm", fq[:, i, :], s) / den
        if return_scale:
            s_abs += fk[:, i, :, None] * np.abs(v[:, i, None, :])
            scale[:, i, :] = np.einsum("bd,bdm->bm", fq[:, i, :], s_abs) / den
    return (out, scale) if return_scale else out
