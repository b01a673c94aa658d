"""Seeded random shapes through every entry point, against the float64 oracle.

Each case draws its sizes (ragged B, T, C, odd widths included), dtype, algorithm, tile length
and input spreads from its own seed, so that combinations the hand-picked cases leave out are
covered: the forward (and the same sequence split in two with the state handed over), the
backward both ways, the gated pair, causal linear attention in both evaluations, and the
token shift with its backward.  Gates are the ones of the dedicated tests: scaled error 2e-5
(float32) / 1e-2 (bf16) for WKV outputs; 5e-5 for gradients, 1e-2 for bf16 dL/dk, dL/dv,
dL/dr; 5e-5 / 1e-2 for linear attention; the token shift's scale-relative 1e-6 / 4e-3.
"""
import numpy as np
import pytest
import torch

from oracle import (scaled_error, token_shift, token_shift_backward, wkv_backward_recurrent,
                    wkv_gated_backward_recurrent, wkv_gated_recurrent, wkv_recurrent)
from oracle.linear_attention import elu_feature, linear_attention_direct
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TORCH_DT, host
from tests.test_backward_gpu import TOL_BF16, TOL_F32, grad_error

pytestmark = pytest.mark.gpu

Y_TOL = {"f32": 2e-5, "bf16": 1e-2}


def dev(a, dtype="f32"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(TORCH_DT[dtype])


def draw_wkv_case(seed):
    rng = np.random.default_rng(7000 + seed)
    dtype = str(rng.choice(["f32", "bf16"]))
    B = int(rng.integers(1, 4))
    T = int(rng.choice([int(rng.integers(1, 130)), int(rng.integers(130, 2600))]))
    C = int(rng.choice([int(rng.integers(1, 70)), int(rng.integers(70, 260))]))
    spec = workloads.FWD_SMALL.with_(B=B, T=T, C=C, dtype=dtype, seed=8000 + seed,
                                     k_std=float(rng.choice([0.5, 1.0, 2.0])),
                                     w_raw_lo=float(rng.choice([-6.0, -3.0])), w_raw_hi=1.0,
                                     u_std=float(rng.choice([0.5, 1.0])))
    algo = str(rng.choice(["auto", "seq", "chunked"]))
    chunk = int(rng.choice([0, 64, 128, 256, 512])) if algo == "chunked" else 0
    return spec, algo, chunk, rng


def grads_ok(got, ref, scale, dtype, names):
    for name, g, r, s in zip(names, got, ref, scale):
        tol = TOL_BF16 if dtype == "bf16" and name in ("gk", "gv", "gr") else TOL_F32
        err = grad_error(g, r, s)
        assert err <= tol, (name, err)


@pytest.mark.parametrize("seed", range(24))
def test_wkv_forward_backward(seed):
    spec, algo, chunk, rng = draw_wkv_case(seed)
    inp = workloads.backward_inputs(spec)
    d = spec.dtype
    w, u = dev(inp["w"]), dev(inp["u"])
    k, v, gy = dev(inp["k"], d), dev(inp["v"], d), dev(inp["gy"], d)
    B, T, C = spec.B, spec.T, spec.C
    print(f"  seed {seed}: {d} B={B} T={T} C={C} {algo} tile {chunk}", flush=True)

    ref, scale = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    y = host(libwkv.wkv_forward(w, u, k, v, algo=algo, chunk_len=chunk))
    assert scaled_error(y, ref, scale) <= Y_TOL[d]

    if T >= 2:  # the same sequence in two calls, the state handed over
        cut = int(rng.integers(1, T))
        y1, st = libwkv.wkv_forward(w, u, k[:, :cut].contiguous(), v[:, :cut].contiguous(), algo=algo,
                                    chunk_len=chunk, return_state=True)
        y2 = libwkv.wkv_forward(w, u, k[:, cut:].contiguous(), v[:, cut:].contiguous(), algo=algo,
                                chunk_len=chunk, state=st)
        split = np.concatenate([host(y1), host(y2)], axis=1)
        assert scaled_error(split, ref, scale) <= Y_TOL[d]

    gref, gscale = wkv_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"], return_scale=True)
    names = ("gw", "gu", "gk", "gv")
    grads_ok([host(g) for g in libwkv.wkv_backward(w, u, k, v, gy)], gref, gscale, d, names)
    y_s, saved = libwkv.wkv_forward_save(w, u, k, v)
    assert scaled_error(host(y_s), ref, scale) <= Y_TOL[d]
    grads_ok([host(g) for g in libwkv.wkv_backward(w, u, k, v, gy, saved=saved)], gref, gscale, d, names)


@pytest.mark.parametrize("seed", range(8))
def test_gated_pair(seed):
    spec, _, _, rng = draw_wkv_case(100 + seed)
    inp = workloads.backward_inputs(spec)
    d = spec.dtype
    r_np = rng.normal(0, 2.0, (spec.B, spec.T, spec.C)).astype(np.float32)
    if d == "bf16":
        r_np = workloads.round_to_bf16(r_np)
    w, u = dev(inp["w"]), dev(inp["u"])
    k, v, gz, r = dev(inp["k"], d), dev(inp["v"], d), dev(inp["gy"], d), dev(r_np, d)
    print(f"  seed {seed}: {d} B={spec.B} T={spec.T} C={spec.C}", flush=True)
    saved = torch.empty(libwkv.wkv_saved_states_bytes(spec.B, spec.T, spec.C), dtype=torch.uint8, device="cuda")
    z = host(libwkv.wkv_forward_gated(w, u, k, v, r, saved=saved))
    zr, zs = wkv_gated_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r_np, return_scale=True)
    assert scaled_error(z, zr, zs) <= Y_TOL[d]
    ref, scale = wkv_gated_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r_np, inp["gy"],
                                              return_scale=True)
    names = ("gw", "gu", "gk", "gv", "gr")
    grads_ok([host(g) for g in libwkv.wkv_backward_gated(w, u, k, v, r, gz, saved=saved)], ref, scale, d, names)
    grads_ok([host(g) for g in libwkv.wkv_backward_gated(w, u, k, v, r, gz)], ref, scale, d, names)


@pytest.mark.parametrize("seed", range(12))
def test_linear_attention(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = str(rng.choice(["f32", "bf16"]))
    D = int(rng.choice([32, 64]))
    spec = workloads.LA_SMALL.with_(BH=int(rng.integers(1, 5)), N=int(rng.integers(1, 1400)), D=D, M=D,
                                    dtype=dtype, seed=9500 + seed)
    feature = bool(rng.integers(0, 2))
    algo = str(rng.choice(["one", "three", "auto"]))
    inp = workloads.linear_attention_inputs(spec)
    if not feature:  # positive features given directly
        for n in ("q", "k"):
            a = np.float32(elu_feature(inp[n]))
            inp[n] = workloads.round_to_bf16(a) if dtype == "bf16" else a
    print(f"  seed {seed}: {dtype} BH={spec.BH} N={spec.N} D={D} feature={feature} {algo}", flush=True)
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    out = host(libwkv.linear_attention(q, k, v, feature_map=feature, algo=algo))
    ref, scale = linear_attention_direct(inp["q"], inp["k"], inp["v"], feature=feature, return_scale=True)
    assert scaled_error(out, ref, scale) <= (5e-5 if dtype == "f32" else 1e-2)


@pytest.mark.parametrize("seed", range(10))
def test_token_shift_pair(seed):
    rng = np.random.default_rng(9900 + seed)
    dtype = str(rng.choice(["f32", "bf16"]))
    B, T, C, M = (int(rng.integers(1, 4)), int(rng.integers(1, 3000)), int(rng.integers(1, 200)),
                  int(rng.integers(1, 5)))
    prev = bool(rng.integers(0, 2))

    def rounded(a):
        a = np.asarray(a, dtype=np.float32)
        return workloads.round_to_bf16(a) if dtype == "bf16" else a

    x = rounded(rng.normal(0, 1, (B, T, C)))
    xp = rounded(rng.normal(0, 1, (B, C))) if prev else None
    mu = rng.uniform(-0.25, 1.25, (M, C)).astype(np.float32)
    g = rounded(rng.normal(0, 1, (M, B, T, C)))
    print(f"  seed {seed}: {dtype} B={B} T={T} C={C} M={M} prev={prev}", flush=True)
    xd, mud, gd = dev(x, dtype), torch.from_numpy(mu).cuda(), dev(g, dtype)
    xpd = None if xp is None else dev(xp, dtype)
    tol = 1e-6 if dtype == "f32" else 4e-3
    x64 = np.asarray(x, dtype=np.float64)
    prev64 = np.zeros((B, 1, C)) if xp is None else np.asarray(xp, dtype=np.float64).reshape(B, 1, C)
    xs = np.concatenate([prev64, x64[:, :-1]], axis=1)  # x_{t-1}
    am, a1m = np.abs(mu)[:, None, None, :], np.abs(1.0 - mu)[:, None, None, :]

    out = host(libwkv.wkv_token_shift(xd, mud, x_prev=xpd))
    scale = am * np.abs(x64)[None] + a1m * np.abs(xs)[None]
    assert np.max(np.abs(out - token_shift(x, mu, xp)) / np.maximum(scale, 1e-30)) <= tol

    gx, gmu, gprev = libwkv.wkv_token_shift_backward(xd, mud, gd, x_prev=xpd)
    rx, rmu, rprev = token_shift_backward(x, mu, g, x_prev=xp)
    g64 = np.asarray(g, dtype=np.float64)
    sx = (am * np.abs(g64)).sum(axis=0)
    sx[:, :-1, :] += (a1m * np.abs(g64[:, :, 1:, :])).sum(axis=0)
    smu = (np.abs(g64) * (np.abs(x64)[None] + np.abs(xs)[None])).sum(axis=2)
    sprev = (np.abs(1.0 - mu)[:, None, :] * np.abs(g64[:, :, 0, :])).sum(axis=0)
    assert np.max(np.abs(host(gx) - rx) / np.maximum(sx, 1e-30)) <= tol
    assert np.max(np.abs(host(gmu) - rmu) / np.maximum(smu, 1e-30)) <= 1e-5
    assert np.max(np.abs(host(gprev) - rprev) / np.maximum(sprev, 1e-30)) <= tol
