"""GPU parity of the token shift and the sigmoid(r) output gate against the float64 oracle.

Gates.  Token shift: |out - ref| / (|mu| |x_t| + |1 - mu| |x_{t-1}|) at most 1e-6 for float32
(one fma and one subtraction) and 4e-3 for bfloat16 (one rounding to bf16, 2^-8 relative at
most).  Gated forward: |z - ref| / (sigmoid(r) s) with s the WKV scale, 2e-5 (float32) and
1e-2 (bfloat16), the forward's gates.  Gated backward: the backward's gates, with the scale of
dL/dr being |gz| s sigmoid(r) sigmoid(-r).
"""
import numpy as np
import pytest
import torch

from oracle import scaled_error, token_shift, token_shift_backward, wkv_gated, wkv_gated_backward
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TORCH_DT, host
from tests.test_backward_gpu import TOL_BF16, TOL_F32, grad_error

pytestmark = pytest.mark.gpu


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(TORCH_DT[dtype])


def rounded(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return workloads.round_to_bf16(a) if dtype == "bf16" else a


# ---- token shift ----

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C,M,prev", [(2, 70, 64, 3, True), (1, 33, 40, 4, False), (3, 5, 7, 1, True),
                                          (1, 1, 8, 2, True), (2, 100, 24, 3, False)])
def test_token_shift(dtype, B, T, C, M, prev):
    rng = np.random.default_rng(B * 100 + T + C + M)
    x = rounded(rng.normal(0, 1, (B, T, C)), dtype)
    xp = rounded(rng.normal(0, 1, (B, C)), dtype) if prev else None
    mu = rng.uniform(-0.25, 1.25, (M, C)).astype(np.float32)
    out = host(libwkv.wkv_token_shift(dev(x, dtype), torch.from_numpy(mu).cuda(),
                                      x_prev=None if xp is None else dev(xp, dtype)))
    ref = token_shift(x, mu, xp)
    xpz = np.zeros((B, 1, C)) if xp is None else xp[:, None, :]
    shifted = np.concatenate([xpz, x[:, :-1]], axis=1)
    scale = np.abs(mu)[:, None, None, :] * np.abs(x)[None] + np.abs(1 - mu)[:, None, None, :] * np.abs(shifted)[None]
    err = scaled_error(out, ref, scale)
    print(f"  token shift {dtype} {B}x{T}x{C} M={M}: {err:.2e}", flush=True)
    assert err <= (1e-6 if dtype == "f32" else 4e-3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_shift_vector_and_element_paths_agree(dtype):
    """16-byte vectors (aligned, C a multiple of the vector) and one element per thread (an
    output that is not 16-byte aligned) do the same arithmetic: bitwise equal."""
    rng = np.random.default_rng(5)
    B, T, C, M = 2, 67, 64, 3
    x = dev(rng.normal(0, 1, (B, T, C)), dtype)
    mu = torch.from_numpy(rng.uniform(0, 1, (M, C)).astype(np.float32)).cuda()
    a = libwkv.wkv_token_shift(x, mu)
    buf = torch.empty(M * B * T * C + 1, dtype=x.dtype, device="cuda")
    b = libwkv.wkv_token_shift(x, mu, out=buf[1:].view(M, B, T, C))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- gated forward ----

def gate_inputs(B, T, C, seed, dtype="f32", **kw):
    inp = workloads.backward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, seed=seed, dtype=dtype, **kw))
    rng = np.random.default_rng(seed + 99)
    inp["r"] = rounded(rng.normal(0, 2.0, (B, T, C)), dtype)
    return inp


def to_dev(inp):
    d = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).cuda() for n in ("w", "u")}
    for n in ("k", "v", "gy", "r"):
        d[n] = dev(inp[n], inp["dtype"])
    return d


@pytest.mark.parametrize("dtype,B,T,C", [("f32", 2, 300, 130), ("f32", 64, 40, 256), ("bf16", 2, 600, 192),
                                         ("bf16", 1, 257, 67), ("f32", 1, 1, 5)])
@pytest.mark.parametrize("save", [False, True])
def test_gated_forward(dtype, B, T, C, save):
    inp = gate_inputs(B, T, C, seed=T + C, dtype=dtype, k_std=1.5)
    d = to_dev(inp)
    saved = None
    if save:
        saved = torch.empty(max(4, libwkv.wkv_saved_states_bytes(B, T, C)), dtype=torch.uint8, device="cuda")
    z = host(libwkv.wkv_forward_gated(d["w"], d["u"], d["k"], d["v"], d["r"], saved=saved))
    ref, scale = wkv_gated(inp["w"], inp["u"], inp["k"], inp["v"], inp["r"], return_scale=True)
    err = scaled_error(z, ref, scale)
    print(f"  gated forward {dtype} {B}x{T}x{C} saved={save}: {err:.2e}", flush=True)
    assert err <= (2e-5 if dtype == "f32" else 1e-2)


def test_bf16_gated_is_rounded_float32_gated():
    """The bf16 gated forward rounds sigma(r) * wkv to bf16 once, from float32 (row pairs too).

    The float32 path on the same bf16-representable inputs gives z32; the bf16 row-pair chunks
    hold 64 tokens per wave against 32 for float32, which changes the float32 rounding of wkv by
    up to about 1e-6 of its scale, so every bf16 output must be the rounding of some float32
    value within 1e-6 * s * sigma(r) of z32 (s: the convex weights applied to |v|), and at
    least 99% of them the rounding of z32 itself.  A gate applied to the bf16-rounded wkv (two
    roundings) misses both."""
    from oracle import wkv_recurrent

    B, T, C = 2, 600, 192
    inp = gate_inputs(B, T, C, seed=77, dtype="bf16", k_std=1.5)
    _, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    sig = 1.0 / (1.0 + np.exp(-inp["r"].astype(np.float64)))
    d16 = to_dev(inp)
    d32 = {n: (t.float() if n in ("k", "v", "r") else t) for n, t in d16.items()}
    for save in (False, True):
        saved = torch.empty(libwkv.wkv_saved_states_bytes(B, T, C), dtype=torch.uint8, device="cuda") if save else None
        z16 = host(libwkv.wkv_forward_gated(d16["w"], d16["u"], d16["k"], d16["v"], d16["r"], saved=saved))
        saved = torch.empty(libwkv.wkv_saved_states_bytes(B, T, C), dtype=torch.uint8, device="cuda") if save else None
        z32 = host(libwkv.wkv_forward_gated(d32["w"], d32["u"], d32["k"], d32["v"], d32["r"], saved=saved))
        d = 1e-6 * s_ref * sig
        lo = workloads.round_to_bf16((z32 - d).astype(np.float32))
        hi = workloads.round_to_bf16((z32 + d).astype(np.float32))
        assert np.all((lo <= z16) & (z16 <= hi)), save
        assert np.mean(z16 == workloads.round_to_bf16(z32)) >= 0.99, save


def test_gated_forward_exact_path():
    """Ill-conditioned waves take the exact per-token path, which applies the gate too."""
    inp = gate_inputs(2, 300, 130, seed=11)
    inp["k"][:, ::37, ::5] = 90.0
    inp["u"][::4] = 70.0
    d = to_dev(inp)
    ref, scale = wkv_gated(inp["w"], inp["u"], inp["k"], inp["v"], inp["r"], return_scale=True)
    for algo_save in (False, True):
        saved = torch.empty(libwkv.wkv_saved_states_bytes(2, 300, 130), dtype=torch.uint8, device="cuda") \
            if algo_save else None
        z = host(libwkv.wkv_forward_gated(d["w"], d["u"], d["k"], d["v"], d["r"], saved=saved))
        assert scaled_error(z, ref, scale) <= 2e-5


# ---- gated backward ----

@pytest.mark.parametrize("dtype,B,T,C", [("f32", 2, 300, 130), ("f32", 1, 700, 64), ("bf16", 2, 400, 128),
                                         ("bf16", 1, 129, 67)])
def test_gated_backward(dtype, B, T, C):
    inp = gate_inputs(B, T, C, seed=T * 3 + C, dtype=dtype)
    d = to_dev(inp)
    got = [host(g) for g in libwkv.wkv_backward_gated(d["w"], d["u"], d["k"], d["v"], d["r"], d["gy"])]
    torch.cuda.synchronize()
    ref, scale = wkv_gated_backward(inp["w"], inp["u"], inp["k"], inp["v"], inp["r"], inp["gy"], return_scale=True)
    for name, g, rr, s in zip(("gw", "gu", "gk", "gv", "gr"), got, ref, scale):
        err = grad_error(g, rr, s)
        tol = TOL_BF16 if dtype == "bf16" and name in ("gk", "gv", "gr") else TOL_F32
        print(f"    {dtype} {B}x{T}x{C} {name}: {err:.3e}", flush=True)
        assert err <= tol, (name, err)


def test_gated_backward_exact_path_and_saved_states():
    inp = gate_inputs(2, 300, 130, seed=12)
    inp["k"][:, 5::41, 1::7] = -90.0
    inp["w"][::3] = -0.05
    d = to_dev(inp)
    ref, scale = wkv_gated_backward(inp["w"], inp["u"], inp["k"], inp["v"], inp["r"], inp["gy"], return_scale=True)
    plain = libwkv.wkv_backward_gated(d["w"], d["u"], d["k"], d["v"], d["r"], d["gy"])
    saved = torch.empty(libwkv.wkv_saved_states_bytes(2, 300, 130), dtype=torch.uint8, device="cuda")
    libwkv.wkv_forward_gated(d["w"], d["u"], d["k"], d["v"], d["r"], saved=saved)
    from_saved = libwkv.wkv_backward_gated(d["w"], d["u"], d["k"], d["v"], d["r"], d["gy"], saved=saved)
    torch.cuda.synchronize()
    for name, a, b, rr, s in zip(("gw", "gu", "gk", "gv", "gr"), plain, from_saved, ref, scale):
        assert torch.equal(a, b), name
        assert grad_error(host(a), rr, s) <= TOL_F32, name


def test_open_gate_gives_the_plain_backward():
    """sigmoid(60) is 1 in float32: dL/dy = gz exactly, so every WKV gradient equals the
    ungated backward's bit for bit, and dL/dr is negligible."""
    inp = gate_inputs(2, 500, 96, seed=13)
    d = to_dev(inp)
    r = torch.full_like(d["k"], 60.0)
    gw, gu, gk, gv, gr = libwkv.wkv_backward_gated(d["w"], d["u"], d["k"], d["v"], r, d["gy"])
    ref = libwkv.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"])
    torch.cuda.synchronize()
    for name, a, b in zip(("gw", "gu", "gk", "gv"), (gw, gu, gk, gv), ref):
        assert torch.equal(a, b), name
    assert float(gr.abs().max()) < 1e-20


# ---- token shift backward ----

SHIFT_BWD_TOL = {"f32": 1e-6, "bf16": 4e-3}


def check_shift_backward(B, T, C, M, dtype, prev, seed, want_gprev=True):
    rng = np.random.default_rng(seed)
    x = rounded(rng.normal(0, 1, (B, T, C)), dtype)
    xp = rounded(rng.normal(0, 1, (B, C)), dtype) if prev else None
    mu = rng.uniform(-0.25, 1.25, (M, C)).astype(np.float32)
    g = rounded(rng.normal(0, 1, (M, B, T, C)), dtype)
    gx, gmu, gprev = libwkv.wkv_token_shift_backward(dev(x, dtype), torch.from_numpy(mu).cuda(), dev(g, dtype),
                                                     x_prev=None if xp is None else dev(xp, dtype),
                                                     want_gprev=want_gprev)
    rx, rmu, rprev = token_shift_backward(x, mu, g, x_prev=xp)
    # scales: the same sums with every term's magnitude
    g64 = np.asarray(g, dtype=np.float64)
    am, a1m = np.abs(mu)[:, None, None, :], np.abs(1.0 - mu)[:, None, None, :]
    sx = (am * np.abs(g64)).sum(axis=0)
    sx[:, :-1, :] += (a1m * np.abs(g64[:, :, 1:, :])).sum(axis=0)
    prev64 = np.zeros((B, 1, C)) if xp is None else np.asarray(xp, dtype=np.float64).reshape(B, 1, C)
    xs = np.concatenate([prev64, np.asarray(x, dtype=np.float64)[:, :-1, :]], axis=1)
    smu = (np.abs(g64) * (np.abs(x)[None] + np.abs(xs)[None])).sum(axis=2)
    sprev = (np.abs(1.0 - mu)[:, None, :] * np.abs(g64[:, :, 0, :])).sum(axis=0)
    err_x = float(np.max(np.abs(host(gx) - rx) / np.maximum(sx, 1e-30)))
    err_mu = float(np.max(np.abs(host(gmu) - rmu) / np.maximum(smu, 1e-30)))
    print(f"  shift bwd B={B} T={T} C={C} M={M} {dtype}: gx {err_x:.2e} gmu {err_mu:.2e}", flush=True)
    assert err_x <= SHIFT_BWD_TOL[dtype], err_x
    assert err_mu <= 1e-5, err_mu  # float32 partials of 32 terms, float64 across segments
    if want_gprev:
        err_p = float(np.max(np.abs(host(gprev) - rprev) / np.maximum(sprev, 1e-30)))
        assert err_p <= SHIFT_BWD_TOL[dtype], err_p
    else:
        assert gprev is None


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C,M,prev", [(2, 70, 64, 3, True), (1, 33, 40, 4, False), (3, 5, 7, 1, True),
                                          (1, 1, 8, 2, True), (2, 100, 24, 3, False), (1, 1000, 130, 3, True),
                                          # 35, 79 and 129 segments of 32 steps: the dL/dmu reduction's eight
                                          # slices of segments are ragged, some empty
                                          (2, 1111, 96, 3, True), (1, 2500, 40, 2, False), (1, 4099, 64, 4, True),
                                          # bf16 vectors of 4 channels (C not a multiple of 8; one mix)
                                          (2, 300, 36, 3, True), (1, 500, 64, 1, False)])
def test_token_shift_backward(dtype, B, T, C, M, prev):
    check_shift_backward(B, T, C, M, dtype, prev, seed=B * 100 + T + C + M)


def test_token_shift_backward_without_gprev_and_empty():
    check_shift_backward(2, 64, 32, 2, "f32", True, seed=5, want_gprev=False)
    x = torch.zeros((2, 0, 16), device="cuda")
    mu = torch.rand((3, 16), device="cuda")
    g = torch.zeros((3, 2, 0, 16), device="cuda")
    gx, gmu, gprev = libwkv.wkv_token_shift_backward(x, mu, g)
    torch.cuda.synchronize()
    assert gmu.shape == (3, 2, 16) and bool((gmu == 0).all()) and bool((gprev == 0).all())
