"""The WKV equation at high precision with mpmath (test infrastructure only).

Page "Reinventing RNNs for the Transformer Era: RWKV" (velog paper review),
section "WKV 연산자", WKV equation: the decayed, normalised weighted average of
v with past weights exp(-(t-1-i) w + k_i) and current weight exp(u + k_t).

Evaluated term by term with ``dps`` significant digits and no rescaling, so it
checks the float64 oracle's rounding on tiny inputs (T up to about 16).
"""
from __future__ import annotations

import mpmath
import numpy as np


def wkv_mp(w, u, k, v, dps=50):
    """Return y [B, T, C] as an object array of mpmath numbers."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nb, T, C = k.shape
    w = np.asarray(w, dtype=np.float64).reshape(C)
    u = np.asarray(u, dtype=np.float64).reshape(C)
    out = np.empty((nb, T, C), dtype=object)
    with mpmath.workdps(dps):
        for bi in range(nb):
            for c in range(C):
                wc = mpmath.mpf(float(w[c]))
                uc = mpmath.mpf(float(u[c]))
                ks = [mpmath.mpf(float(x)) for x in k[bi, :, c]]
                vs = [mpmath.mpf(float(x)) for x in v[bi, :, c]]
                for t in range(T):
                    num = mpmath.mpf(0)
                    den = mpmath.mpf(0)
                    for i in range(t):
                        e = mpmath.exp(-(t - 1 - i) * wc + ks[i])
                        num += e * vs[i]
                        den += e
                    e = mpmath.exp(uc + ks[t])
                    num += e * vs[t]
                    den += e
                    out[bi, t, c] = num / den
    return out
