"""The training-side calls at the full sizes the benchmark times, every element against the
float64 oracle's O(T) forms (themselves pinned to the O(T^2) definitions without a GPU).

Workloads: B=8, T=8192, C=2048 float32 (the 8K-context, 1.5B-width layer) and B=1, T=65536,
C=5120 bf16 (64K tokens at 14B width), seeded NumPy inputs (workloads.backward_inputs, with
the gate r ~ N(0, 2) and the token-shift mixes mu ~ U(0, 1) from their own seeded streams).
Calls: wkv_backward (recomputing forward), wkv_forward_save + wkv_backward_saved,
wkv_forward_gated + wkv_backward_gated, wkv_token_shift with three mixes and its backward
(dL/dout ~ N(0, 1) from its own seeded stream).  Gates as in the
smaller tests: gradients 5e-5 (float32; gw, gu always) and 1e-2 (bf16 gk, gv, gr), the forward's
2e-5 / 1e-2, the token shift's 1e-6 / 4e-3 of |mu x_t| + |(1 - mu) x_{t-1}|.
"""
import numpy as np
import pytest
import torch

from oracle import scaled_error, token_shift, token_shift_backward, wkv_backward_recurrent, \
    wkv_gated_backward_recurrent, wkv_gated_recurrent
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TOL, TORCH_DT, host
from tests.test_backward_gpu import TOL_BF16, TOL_F32, grad_error

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SHIFT_TOL = {"f32": 1e-6, "bf16": 4e-3}


def gate_and_mix(spec):
    rng = np.random.default_rng(spec.seed + 5_555_555)
    r = rng.standard_normal(size=(spec.B, spec.T, spec.C), dtype=np.float32)
    r *= np.float32(2.0)
    if spec.dtype == "bf16":
        r = workloads.round_to_bf16(r)
    mu = rng.uniform(0.0, 1.0, size=(3, spec.C)).astype(np.float32)
    return r, mu


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda().to(TORCH_DT[dtype])


def check_grads(label, got, ref, scale, dtype, names=("gw", "gu", "gk", "gv")):
    """got: host float64 arrays."""
    for name, g, rr, s in zip(names, got, ref, scale):
        err = grad_error(g, rr, s)
        tol = TOL_BF16 if dtype == "bf16" and name in ("gk", "gv", "gr") else TOL_F32
        print(f"  {label} {name}: scaled error {err:.3e}", flush=True)
        assert err <= tol, (label, name, err)


def run_training_calls(spec):
    dt = spec.dtype
    print(f"  {spec.name}: generating", flush=True)
    inp = workloads.backward_inputs(spec)
    r, mu = gate_and_mix(spec)
    w, u = (torch.from_numpy(inp[n]).cuda() for n in ("w", "u"))
    k, v, gy, rd = (to_dev(x, dt) for x in (inp["k"], inp["v"], inp["gy"], r))
    B, T, C = spec.B, spec.T, spec.C

    # GPU calls first (host copies kept), then the device memory is released for the oracle
    ws = libwkv.new_backward_workspace(B, T, C, k.dtype)
    g_plain = [host(x) for x in libwkv.wkv_backward(w, u, k, v, gy, workspace=ws)]
    assert libwkv.lookback_error(ws) == 0
    fws = libwkv.new_workspace(B, T, C, k.dtype, "chunked", 0)
    y_save, saved = libwkv.wkv_forward_save(w, u, k, v, workspace=fws)
    g_saved = [host(x) for x in libwkv.wkv_backward(w, u, k, v, gy, saved=saved, workspace=ws)]
    assert libwkv.lookback_error(fws) == 0 and libwkv.lookback_error(ws) == 0
    y_save = host(y_save)
    del saved
    z = host(libwkv.wkv_forward_gated(w, u, k, v, rd, workspace=libwkv.new_workspace(B, T, C, k.dtype)))
    g_gated = [host(x) for x in libwkv.wkv_backward_gated(w, u, k, v, rd, gy, workspace=ws)]
    assert libwkv.lookback_error(ws) == 0
    shift = host(libwkv.wkv_token_shift(k, torch.from_numpy(mu).cuda()))
    gs = np.random.default_rng(spec.seed + 3_333_333).standard_normal(size=(3, B, T, C), dtype=np.float32)
    if dt == "bf16":
        gs = workloads.round_to_bf16(gs)
    sb = [host(x) for x in libwkv.wkv_token_shift_backward(k, torch.from_numpy(mu).cuda(), to_dev(gs, dt))]
    del k, v, gy, rd, ws, fws
    torch.cuda.empty_cache()
    print(f"  {spec.name}: GPU calls done", flush=True)

    # token shift: x = k (already rounded to the dtype)
    ts_ref = token_shift(inp["k"], mu)
    prev = np.concatenate([np.zeros((B, 1, C)), inp["k"][:, :-1, :].astype(np.float64)], axis=1)
    ts_scale = np.abs(mu)[:, None, None, :] * np.abs(inp["k"])[None] + \
        np.abs(1.0 - mu)[:, None, None, :] * np.abs(prev)[None]
    err = float(np.max(np.abs(shift - ts_ref) / np.maximum(ts_scale, 1e-30)))
    print(f"  {spec.name} token shift x3: {err:.3e}", flush=True)
    assert err <= SHIFT_TOL[dt], err
    del ts_ref, ts_scale, shift
    # its backward: dL/dx against the same sums of magnitudes, dL/dmu per lane likewise
    rx, rmu, rprev = token_shift_backward(inp["k"], mu, gs)
    g64 = np.abs(gs.astype(np.float64))
    sx = (np.abs(mu)[:, None, None, :] * g64).sum(axis=0)
    sx[:, :-1, :] += (np.abs(1.0 - mu)[:, None, None, :] * g64[:, :, 1:, :]).sum(axis=0)
    err_x = float(np.max(np.abs(sb[0] - rx) / np.maximum(sx, 1e-30)))
    smu = (g64 * (np.abs(inp["k"])[None] + np.abs(prev)[None])).sum(axis=2)
    err_mu = float(np.max(np.abs(sb[1] - rmu) / np.maximum(smu, 1e-30)))
    print(f"  {spec.name} token shift backward: gx {err_x:.3e} gmu {err_mu:.3e}", flush=True)
    assert err_x <= SHIFT_TOL[dt] and err_mu <= 1e-5, (err_x, err_mu)
    del rx, rmu, rprev, g64, sx, smu, sb, gs, prev

    # plain backward and the saved pair against the reverse recurrence
    ref, scale = wkv_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"], return_scale=True)
    print(f"  {spec.name}: gradient oracle done", flush=True)
    check_grads("wkv_backward", g_plain, ref, scale, dt)
    check_grads("wkv_backward_saved", g_saved, ref, scale, dt)
    del ref, scale, g_plain, g_saved

    # gated pair (the forward_save output is checked through the gated oracle's y: z / sigmoid(r))
    z_ref, sz = wkv_gated_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r, return_scale=True)
    err = scaled_error(z, z_ref, sz)
    print(f"  {spec.name} wkv_forward_gated: {err:.3e}", flush=True)
    assert err <= TOL[dt], err
    del z_ref, sz, z
    gref, gscale = wkv_gated_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r, inp["gy"],
                                                return_scale=True)
    check_grads("wkv_backward_gated", g_gated, gref, gscale, dt, names=("gw", "gu", "gk", "gv", "gr"))
    del gref, gscale
    from oracle import wkv_recurrent
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    err = scaled_error(y_save, y_ref, s_ref)
    print(f"  {spec.name} wkv_forward_save: {err:.3e}", flush=True)
    assert err <= TOL[dt], err


@pytest.mark.timeout(900)
def test_training_calls_ctx8192_width2048_f32():
    run_training_calls(workloads.FWD_CTX8K)


@pytest.mark.timeout(1200)
def test_training_calls_ctx65536_width5120_bf16():
    run_training_calls(workloads.FWD_LONG_BF16)


@pytest.mark.timeout(600)
def test_backward_bf16_long_sequence():
    """bf16 backward over 24,000 tokens (188 tiles of 128 chained backwards), every element."""
    spec = workloads.FWD_LONG_BF16.with_(B=2, T=24000, C=192, seed=7)
    inp = workloads.backward_inputs(spec)
    w, u = (torch.from_numpy(inp[n]).cuda() for n in ("w", "u"))
    k, v, gy = (to_dev(inp[n], "bf16") for n in ("k", "v", "gy"))
    ws = libwkv.new_backward_workspace(spec.B, spec.T, spec.C, k.dtype)
    got = [host(x) for x in libwkv.wkv_backward(w, u, k, v, gy, workspace=ws)]
    assert libwkv.lookback_error(ws) == 0
    ref, scale = wkv_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"], return_scale=True)
    check_grads("bf16 T=24000", got, ref, scale, "bf16")
