"""Every wrapper run on a side stream (``stream=``) while torch's current stream is held busy.

The wrappers allocate their outputs and workspaces, and zero-fill the workspaces, on the stream
they launch on (the binding's ``_on_stream``).  Here the current stream spins for a few milliseconds or more
after the inputs are made, and the call goes to another stream that only waits for the
inputs: a fill or an allocation ordered on the current stream instead would land after the
launch that needs it.  Each result must match the float64 oracle at the usual gates and be
bitwise the result of the same call on the current stream (the kernels are deterministic).
"""
import contextlib

import numpy as np
import pytest
import torch

from oracle import (linear_attention_direct, scaled_error, token_shift, token_shift_backward,
                    wkv_backward_recurrent, wkv_gated_backward_recurrent, wkv_gated_recurrent, wkv_recurrent)
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TORCH_DT, host
from tests.test_backward_gpu import TOL_BF16, TOL_F32, grad_error

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 10_000_000  # torch.cuda._sleep cycles: a few ms (shader clock) to 0.1 s (100 MHz counter)


def dev(a, dtype="f32"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(TORCH_DT[dtype])


def on_side_stream(call):
    """call(stream) on a fresh side stream that waits for the inputs only, with the current
    stream spinning meanwhile; returns the result after both streams are done."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    torch.cuda._sleep(SPIN_CYCLES)  # the current stream is busy from here on
    out = call(side)
    torch.cuda.synchronize()
    return out


def stream_ctx(s):
    """Allocations the caller makes for a call on stream s come from s."""
    return torch.cuda.stream(s) if s is not None else contextlib.nullcontext()


def as_host(out):
    if isinstance(out, (tuple, list)):
        return [as_host(x) for x in out]
    return host(out)


def same_bits(a, b):
    if isinstance(a, (tuple, list)):
        return all(same_bits(x, y) for x, y in zip(a, b))
    return np.array_equal(np.asarray(a), np.asarray(b), equal_nan=True)


def forward_inputs(B, T, C, dtype, seed):
    return workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, dtype=dtype, seed=seed))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward(dtype):
    inp = forward_inputs(2, 1500, 96, dtype, seed=21)
    w, u, k, v = dev(inp["w"]), dev(inp["u"]), dev(inp["k"], dtype), dev(inp["v"], dtype)
    here = host(libwkv.wkv_forward(w, u, k, v, algo="chunked"))
    side = host(on_side_stream(lambda s: libwkv.wkv_forward(w, u, k, v, algo="chunked", stream=s)))
    ref, scale = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    assert scaled_error(side, ref, scale) <= (2e-5 if dtype == "f32" else 1e-2)
    assert same_bits(side, here)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_and_training_pair(dtype):
    spec = workloads.FWD_SMALL.with_(B=2, T=900, C=64, dtype=dtype, seed=22)
    inp = workloads.backward_inputs(spec)
    w, u, k, v, gy = (dev(inp["w"]), dev(inp["u"]), dev(inp["k"], dtype), dev(inp["v"], dtype),
                      dev(inp["gy"], dtype))
    ref, scale = wkv_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"], return_scale=True)

    def pair(s=None):
        _, saved = libwkv.wkv_forward_save(w, u, k, v, stream=s)
        return libwkv.wkv_backward(w, u, k, v, gy, saved=saved, stream=s)

    for fn in (lambda s=None: libwkv.wkv_backward(w, u, k, v, gy, stream=s), pair):
        here = as_host(fn())
        side = as_host(on_side_stream(lambda s: fn(s)))
        for name, g, r, sc in zip(("gw", "gu", "gk", "gv"), side, ref, scale):
            tol = TOL_BF16 if dtype == "bf16" and name in ("gk", "gv") else TOL_F32
            assert grad_error(g, r, sc) <= tol, name
        assert same_bits(side, here)


def test_gated_pair():
    spec = workloads.FWD_SMALL.with_(B=2, T=700, C=64, seed=23)
    inp = workloads.backward_inputs(spec)
    r_np = np.random.default_rng(23).normal(0, 1, inp["k"].shape).astype(np.float32)
    w, u, k, v, gz, r = (dev(inp["w"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), dev(inp["gy"]), dev(r_np))

    def gated(s=None):
        with stream_ctx(s):
            saved = torch.empty(libwkv.wkv_saved_states_bytes(2, 700, 64), dtype=torch.uint8, device="cuda")
        z = libwkv.wkv_forward_gated(w, u, k, v, r, saved=saved, stream=s)
        return (z,) + tuple(libwkv.wkv_backward_gated(w, u, k, v, r, gz, saved=saved, stream=s))

    here = as_host(gated())
    side = as_host(on_side_stream(lambda s: gated(s)))
    zr, zs = wkv_gated_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r_np, return_scale=True)
    assert scaled_error(side[0], zr, zs) <= 2e-5
    ref, scale = wkv_gated_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r_np, inp["gy"],
                                              return_scale=True)
    for name, g, rr, sc in zip(("gw", "gu", "gk", "gv", "gr"), side[1:], ref, scale):
        assert grad_error(g, rr, sc) <= TOL_F32, name
    assert same_bits(side, here)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linear_attention(dtype):
    spec = workloads.LA_SMALL.with_(BH=6, N=1300, dtype=dtype, seed=24)
    inp = workloads.linear_attention_inputs(spec)
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    here = host(libwkv.linear_attention(q, k, v, algo="one"))
    side = host(on_side_stream(lambda s: libwkv.linear_attention(q, k, v, algo="one", stream=s)))
    ref, scale = linear_attention_direct(inp["q"], inp["k"], inp["v"], return_scale=True)
    assert scaled_error(side, ref, scale) <= (5e-5 if dtype == "f32" else 1e-2)
    assert same_bits(side, here)


def test_token_shift_and_backward():
    rng = np.random.default_rng(25)
    x = rng.normal(0, 1, (2, 300, 64)).astype(np.float32)
    xp = rng.normal(0, 1, (2, 64)).astype(np.float32)
    mu = rng.uniform(0, 1, (3, 64)).astype(np.float32)
    g = rng.normal(0, 1, (3, 2, 300, 64)).astype(np.float32)
    xd, xpd, mud, gd = dev(x), dev(xp), torch.from_numpy(mu).cuda(), dev(g)

    def both(s=None):
        out = libwkv.wkv_token_shift(xd, mud, x_prev=xpd, stream=s)
        return (out,) + tuple(libwkv.wkv_token_shift_backward(xd, mud, gd, x_prev=xpd, stream=s))

    here = as_host(both())
    side = as_host(on_side_stream(lambda s: both(s)))
    ref = token_shift(x, mu, xp)
    scale = np.abs(mu)[:, None, None, :] * np.abs(x)[None] + np.abs(1 - mu)[:, None, None, :] * np.abs(
        np.concatenate([xp[:, None], x[:, :-1]], axis=1))[None]
    assert np.max(np.abs(side[0] - ref) / np.maximum(scale, 1e-30)) <= 1e-6
    rgx, rgmu, rgp = token_shift_backward(x, mu, g, x_prev=xp)
    for got, want in zip(side[1:], (rgx, rgmu, rgp)):
        assert np.max(np.abs(got - want)) <= 1e-4 * max(1.0, np.max(np.abs(want)))
    assert same_bits(side, here)


def test_step():
    rng = np.random.default_rng(26)
    N, G, C = 8, 2, 64
    w = torch.from_numpy(np.exp(rng.uniform(-3, 1, (G, C))).astype(np.float32)).cuda()
    u = torch.from_numpy(rng.normal(0, 0.5, (G, C)).astype(np.float32)).cuda()
    kv = [(dev(rng.normal(0, 1, (N, G, C))), dev(rng.normal(0, 1, (N, G, C)))) for _ in range(5)]

    def decode(s=None):
        with stream_ctx(s):
            a, b, p = libwkv.empty_state((N, G, C))
        ys = [libwkv.wkv_step(w, u, k, v, a, b, p, stream=s) for k, v in kv]
        return ys + [a, b, p]

    here = as_host(decode())
    side = as_host(on_side_stream(lambda s: decode(s)))
    assert same_bits(side, here)
