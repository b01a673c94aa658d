"""The chained scans' give-up path, forced from the host, against the float64 oracle.

A tile whose wait gives up rebuilds the state it needs without waiting: from the nearest
complete inclusive record (or the sequence's start / end), through the complete aggregate
records after it, re-reading the inputs of any tile whose record is missing.  The test hook
wkv_workspace_force_give_up makes every tile of the next launches take that path at once, so
every kernel still exits normally; outputs must meet the same gates as the usual path, and the
workspace must report the give-up.  Gates: the forward's 2e-5 (float32) and 1e-2 (bf16), the
backward's 5e-5 / 1e-2 (gradients), linear attention's 5e-5 / 1e-2.
"""
import numpy as np
import pytest
import torch

from oracle import scaled_error, wkv_backward_recurrent, wkv_gated_backward_recurrent, wkv_gated_recurrent, \
    wkv_recurrent
from oracle.linear_attention import linear_attention_recurrent
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TOL, TORCH_DT, host, to_device
from tests.test_backward_gpu import TOL_BF16, TOL_F32, grad_error

pytestmark = pytest.mark.gpu


def fwd_inputs(B, T, C, dtype="f32", seed=3, **kw):
    return workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, dtype=dtype, seed=seed, **kw))


@pytest.mark.parametrize("dtype,B,T,C,chunk", [("f32", 2, 3000, 130, 256), ("f32", 1, 5000, 64, 128),
                                               ("bf16", 2, 4100, 128, 512), ("bf16", 1, 3000, 67, 256),
                                               ("f32", 3, 700, 200, 64), ("f32", 4, 40000, 128, 128),
                                               ("bf16", 2, 40000, 256, 512)])
def test_forward_forced(dtype, B, T, C, chunk):
    """Every tile rebuilds its entering state; the next call on the workspace is back on the usual path.
    The first five launches fit on the GPU at once (tiles numbered by workgroup index); the last two
    have 2504 and 632 tiles, more than fit, and take tickets."""
    inp = fwd_inputs(B, T, C, dtype, seed=B + T + C, k_std=1.5)
    dev = to_device(inp)
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    k = dev["k"]
    ws = libwkv.new_workspace(B, T, C, k.dtype, "chunked", chunk)
    libwkv.force_give_up(ws, 1)
    y = libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo="chunked", chunk_len=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 1
    err = scaled_error(host(y), y_ref, s_ref)
    print(f"  forced {dtype} B={B} T={T} C={C} chunk={chunk}: {err:.2e}", flush=True)
    assert err <= TOL[dtype], err
    y = libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo="chunked", chunk_len=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 0
    assert scaled_error(host(y), y_ref, s_ref) <= TOL[dtype]


def test_forward_forced_with_state():
    """State in and out through the rebuilt path (the rebuild starts from the state in)."""
    B, T, C = 2, 2600, 96
    inp = fwd_inputs(B, T, C, seed=17)
    rng = np.random.default_rng(5)
    a0 = rng.normal(0, 1, (B, C)).astype(np.float32)
    b0 = rng.uniform(0.5, 2.0, (B, C)).astype(np.float32)
    p0 = rng.normal(0, 3, (B, C)).astype(np.float32)
    # the state's own |v| weight is taken as |a| (a lower bound of what it summed), so the scale
    # still bounds every output
    y_ref, s_ref, (ra, rb, rp) = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"],
                                               state=(a0, b0, p0, np.abs(a0)), return_scale=True,
                                               return_state=True)
    dev = to_device(inp)
    st = tuple(torch.from_numpy(x).cuda() for x in (a0, b0, p0))
    ws = libwkv.new_workspace(B, T, C, torch.float32, "chunked", 256)
    libwkv.force_give_up(ws, 1)
    y, (oa, ob, op) = libwkv.wkv_forward(dev["w"], dev["u"], dev["k"], dev["v"], algo="chunked", chunk_len=256,
                                         workspace=ws, state=st, return_state=True)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 1
    err = scaled_error(host(y), y_ref, s_ref)
    assert err <= TOL["f32"], err
    np.testing.assert_allclose(host(op) + np.log(host(ob)), rp + np.log(rb), rtol=0, atol=2e-5)


def bwd_inputs(B, T, C, dtype="f32", seed=0, **kw):
    return workloads.backward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, seed=seed, dtype=dtype, **kw))


def bdev(inp):
    dt = TORCH_DT[inp["dtype"]]
    d = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).cuda() for n in ("w", "u")}
    for n in ("k", "v", "gy"):
        d[n] = torch.from_numpy(np.ascontiguousarray(inp[n])).cuda().to(dt)
    return d


def check_grads(got, inp):
    ref, scale = wkv_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"], return_scale=True)
    for name, g, r, s in zip(("gw", "gu", "gk", "gv"), got, ref, scale):
        err = grad_error(g, r, s)
        tol = TOL_BF16 if inp["dtype"] == "bf16" and name in ("gk", "gv") else TOL_F32
        print(f"    {name}: {err:.2e}", flush=True)
        assert err <= tol, (name, err)


@pytest.mark.parametrize("dtype,B,T,C", [("f32", 2, 2000, 130), ("bf16", 1, 3000, 128), ("bf16", 2, 1500, 67)])
def test_backward_forced(dtype, B, T, C):
    """wkv_backward recomputes the forward states (one launch) then scans backwards (another):
    both are forced onto the rebuild path."""
    inp = bwd_inputs(B, T, C, dtype, seed=T + C, k_std=1.5)
    d = bdev(inp)
    ws = libwkv.new_backward_workspace(B, T, C, d["k"].dtype)
    libwkv.force_give_up(ws, 2)
    got = libwkv.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], workspace=ws)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 1
    check_grads([host(x) for x in got], inp)


def test_training_pair_forced():
    """wkv_forward_save and wkv_backward_saved, each forced."""
    B, T, C = 2, 2500, 96
    inp = bwd_inputs(B, T, C, "f32", seed=44)
    d = bdev(inp)
    fws = libwkv.new_workspace(B, T, C, torch.float32, "chunked", 0)
    bws = libwkv.new_backward_workspace(B, T, C, torch.float32)
    libwkv.force_give_up(fws, 1)
    y, saved = libwkv.wkv_forward_save(d["w"], d["u"], d["k"], d["v"], workspace=fws)
    libwkv.force_give_up(bws, 1)
    got = libwkv.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], saved=saved, workspace=bws)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(fws) == 1 and libwkv.lookback_error(bws) == 1
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    assert scaled_error(host(y), y_ref, s_ref) <= TOL["f32"]
    check_grads([host(x) for x in got], inp)


def test_gated_pair_forced():
    """The gated forward and backward (dL/dr too), each forced."""
    B, T, C = 1, 2200, 128
    inp = bwd_inputs(B, T, C, "f32", seed=45)
    r = np.random.default_rng(46).normal(0, 2, (B, T, C)).astype(np.float32)
    d = bdev(inp)
    rd = torch.from_numpy(r).cuda()
    fws = libwkv.new_workspace(B, T, C, torch.float32, "auto", 0)
    if fws is not None:
        libwkv.force_give_up(fws, 1)
    z = libwkv.wkv_forward_gated(d["w"], d["u"], d["k"], d["v"], rd, workspace=fws)
    bws = libwkv.new_backward_workspace(B, T, C, torch.float32)
    libwkv.force_give_up(bws, 2)
    got = libwkv.wkv_backward_gated(d["w"], d["u"], d["k"], d["v"], rd, d["gy"], workspace=bws)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(bws) == 1
    z_ref, sz = wkv_gated_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r, return_scale=True)
    assert scaled_error(host(z), z_ref, sz) <= TOL["f32"]
    ref, scale = wkv_gated_backward_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], r, inp["gy"],
                                              return_scale=True)
    for name, g, rr, s in zip(("gw", "gu", "gk", "gv", "gr"), got, ref, scale):
        err = grad_error(host(g), rr, s)
        print(f"    {name}: {err:.2e}", flush=True)
        assert err <= TOL_F32, (name, err)


@pytest.mark.parametrize("dtype,BH,N,D", [("f32", 4, 3000, 32), ("bf16", 3, 5000, 32), ("f32", 2, 1500, 64)])
def test_linear_attention_forced(dtype, BH, N, D):
    spec = workloads.LA_SMALL.with_(BH=BH, N=N, D=D, M=D, dtype=dtype, seed=N)
    inp = workloads.linear_attention_inputs(spec)
    dt = TORCH_DT[dtype]
    q, k, v = (torch.from_numpy(inp[n]).cuda().to(dt) for n in ("q", "k", "v"))
    ws = libwkv.new_la_workspace(BH, N, D, D, dt)
    libwkv.force_give_up(ws, 1)
    out = libwkv.linear_attention(q, k, v, workspace=ws, algo="one")
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 1
    ref, scale = linear_attention_recurrent(inp["q"], inp["k"], inp["v"], return_scale=True)
    err = scaled_error(host(out), ref, scale)
    print(f"  forced linear attention {dtype} BH={BH} N={N} D={D}: {err:.2e}", flush=True)
    assert err <= {"f32": 5e-5, "bf16": 1e-2}[dtype], err
