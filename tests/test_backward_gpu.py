"""GPU parity of wkv_backward against the float64 gradient oracle.

Gate: per element, |g_gpu - g| / s where s is the same sum the oracle forms with
every term replaced by its magnitude (|gy|, and |v_i| + |y_t| for v_i - y_t), so
the bound is a relative error wherever the terms share a sign.  The scale is
floored at 2^-100 of its largest value in the tensor: below that, float32
products of the kernel may flush to zero, and such gradients carry no weight.

Bounds.  float32: 5e-5.  Every gradient is a float32 sum of positive-weight terms
(with magnitudes exactly those of the scale); each term carries the forward's
error (the forward's own gate is 2e-5) and each fold of a reverse carry or of a
partial sum adds a few roundings -- 16 tokens per wave, 8 waves per tile and one
fold per 128-token tile, about 2e-6 at T = 4096.  bfloat16 k, v, gy: gk and gv
are rounded to bfloat16 once (relative 2^-9) and take the forward's 1e-2; gw and
gu stay float32 and keep the float32 bound.
"""
import numpy as np
import pytest
import torch

from oracle import wkv_backward_direct
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TORCH_DT, host

pytestmark = pytest.mark.gpu

TOL_F32 = 5e-5
TOL_BF16 = 1e-2
NAMES = ("gw", "gu", "gk", "gv")


def grad_error(got, ref, scale):
    got, ref, scale = (np.asarray(x, dtype=np.float64) for x in (got, ref, scale))
    if scale.size == 0:
        return 0.0
    s = np.maximum(scale, 2.0 ** -100 * scale.max())
    err = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s == 0, np.where(err == 0, 0.0, np.inf), err / np.where(s == 0, 1.0, s))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    return float(ratio.max())


def to_device(inp):
    dt = TORCH_DT[inp["dtype"]]
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).cuda() for n in ("w", "u")}
    for n in ("k", "v", "gy"):
        dev[n] = torch.from_numpy(np.ascontiguousarray(inp[n])).cuda().to(dt)
    return dev


def run_backward(dev, workspace=None):
    B, T, C = dev["k"].shape
    ws = workspace
    if ws is None:
        ws = libwkv.new_backward_workspace(B, T, C, dev["k"].dtype, device=dev["k"].device)
    out = libwkv.wkv_backward(dev["w"], dev["u"], dev["k"], dev["v"], dev["gy"], workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert libwkv.lookback_error(ws) == 0, "a scan gave up waiting"
    return [host(x) for x in out]


def check(inp, label=""):
    B, T, C = inp["k"].shape
    print(f"  {label} B={B} T={T} C={C} {inp['dtype']}", flush=True)
    ref, scale = wkv_backward_direct(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"], return_scale=True)
    got = run_backward(to_device(inp))
    for name, g, r, s in zip(NAMES, got, ref, scale):
        err = grad_error(g, r, s)
        tol = TOL_BF16 if inp["dtype"] == "bf16" and name in ("gk", "gv") else TOL_F32
        print(f"    {name}: scaled error {err:.3e}", flush=True)
        assert err <= tol, (label, name, err)
    return got


def grad_inputs(B, T, C, seed=0, dtype="f32", **kw):
    return workloads.backward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, seed=seed, dtype=dtype, **kw))


def test_small_workload():
    """B=1, T=64, C=64 float32."""
    check(workloads.backward_inputs(workloads.FWD_SMALL), "small")


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 1, 7), (1, 2, 3), (1, 15, 5), (1, 17, 64), (3, 127, 100),
                                   (2, 129, 65), (1, 257, 130), (2, 300, 64), (1, 700, 1)])
def test_ragged_shapes(B, T, C):
    check(grad_inputs(B, T, C, seed=B * 1000 + T + C), "ragged")


def test_tile_boundaries():
    """T around the 128-token tile and its 16-token waves, several tiles."""
    for T in (16, 112, 127, 128, 129, 144, 389, 512):
        check(grad_inputs(2, T, 70, seed=T, k_std=1.5), f"T={T}")


def test_many_tiles():
    """32 tiles per lane: the reverse carry crosses every tile boundary."""
    check(grad_inputs(1, 4096, 64, seed=5, k_std=1.5, w_raw_lo=-6.0), "many tiles")


def test_bf16_io():
    """bfloat16 k, v, gy, gk, gv (float32 gw, gu), even and odd C."""
    check(grad_inputs(2, 300, 128, seed=21, dtype="bf16"), "bf16")
    check(grad_inputs(1, 260, 67, seed=22, dtype="bf16"), "bf16 odd C")


@pytest.mark.parametrize("case", ["negative_w", "huge_k_range", "huge_u", "tiny_u", "w_zero", "k_plus_200",
                                  "k_minus_200", "sparse_gy"])
def test_exact_fallback_cases(case):
    """Inputs outside the fast path's conditioning run the exact per-token path."""
    inp = grad_inputs(2, 300, 130, seed=11)
    if case == "negative_w":
        inp["w"][::3] = -0.05
    elif case == "huge_k_range":
        inp["k"][:, ::37, ::5] = 90.0
        inp["k"][:, 5::41, 1::7] = -90.0
    elif case == "huge_u":
        inp["u"][::4] = 70.0
    elif case == "tiny_u":
        inp["u"][::4] = -70.0
    elif case == "w_zero":
        inp["w"][:] = 0.0
    elif case == "k_plus_200":
        inp["k"] = (inp["k"].astype(np.float64) + 200.0).astype(np.float32)
    elif case == "k_minus_200":
        inp["k"] = (inp["k"].astype(np.float64) - 200.0).astype(np.float32)
    elif case == "sparse_gy":  # the reverse carry is empty over long stretches
        inp["gy"][:, 20:290] = 0.0
    check(inp, case)


def test_zero_gy_gives_zero_gradients():
    inp = grad_inputs(2, 300, 96, seed=3)
    inp["gy"][:] = 0.0
    for name, g in zip(NAMES, run_backward(to_device(inp))):
        assert np.all(g == 0.0), name


def test_empty_sequence_zeroes_w_u_gradients():
    gw = torch.full((2, 5), 7.0, device="cuda")
    gu = torch.full((2, 5), 7.0, device="cuda")
    z = torch.empty((2, 0, 5), device="cuda")
    w = torch.ones(5, device="cuda")
    libwkv.wkv_backward(w, w, z, z, z, gw=gw, gu=gu)
    torch.cuda.synchronize()
    assert torch.all(gw == 0) and torch.all(gu == 0)


def test_deterministic_and_workspace_reuse():
    """Bitwise-equal gradients from repeated calls; one workspace serves a smaller problem too."""
    inp = grad_inputs(3, 1000, 200, seed=4, k_std=2.0)
    dev = to_device(inp)
    ws = libwkv.new_backward_workspace(3, 1000, 200)
    first = run_backward(dev, ws)
    for _ in range(2):
        again = run_backward(dev, ws)
        for name, a, b in zip(NAMES, first, again):
            assert np.array_equal(a, b), name
    small = grad_inputs(1, 200, 64, seed=8)
    ref, scale = wkv_backward_direct(small["w"], small["u"], small["k"], small["v"], small["gy"], return_scale=True)
    got = run_backward(to_device(small), ws)
    for name, g, r, s in zip(NAMES, got, ref, scale):
        assert grad_error(g, r, s) <= TOL_F32, name


def test_channel_gradient_is_batch_sum():
    """Summing the per-lane gw, gu over the batch gives the [C] parameters' gradients:
    checked against the oracle's per-lane sums (the oracle's pin to finite
    differences covers the summed form)."""
    inp = grad_inputs(4, 200, 64, seed=6)
    ref = wkv_backward_direct(inp["w"], inp["u"], inp["k"], inp["v"], inp["gy"])
    gw, gu, _, _ = run_backward(to_device(inp))
    np.testing.assert_allclose(gw.sum(0), ref[0].sum(0), rtol=1e-4, atol=1e-4 * np.abs(ref[0]).max())
    np.testing.assert_allclose(gu.sum(0), ref[1].sum(0), rtol=1e-4, atol=1e-4 * np.abs(ref[1]).max())


def test_long_sequence_sampled_lanes():
    """T = 20000 (157 tiles): sampled lanes against the oracle run on those lanes alone."""
    spec = workloads.FWD_SMALL.with_(B=2, T=20000, C=130, k_std=1.5, w_raw_lo=-6.0, seed=12)
    inp = workloads.backward_inputs(spec)
    got = run_backward(to_device(inp))
    for (b, c) in workloads.sample_lanes(spec.B, spec.C, 3, seed=2):
        sl = {n: inp[n][b:b + 1, :, c:c + 1] for n in ("k", "v", "gy")}
        ref, scale = wkv_backward_direct(inp["w"][c:c + 1], inp["u"][c:c + 1], sl["k"], sl["v"], sl["gy"],
                                         return_scale=True)
        for i, name in enumerate(NAMES):
            g = got[i][b:b + 1, c:c + 1] if i < 2 else got[i][b:b + 1, :, c:c + 1]
            err = grad_error(g, ref[i], scale[i])
            print(f"    lane ({b},{c}) {name}: {err:.3e}", flush=True)
            assert err <= TOL_F32, (b, c, name, err)


def test_workspace_epoch_advances_twice_per_call():
    """Each call runs two chained scans on the workspace's control block (forward, then
    backward in time); neither gives up."""
    inp = grad_inputs(2, 1000, 130, seed=13)
    dev = to_device(inp)
    ws = libwkv.new_backward_workspace(2, 1000, 130)
    for i in range(3):
        run_backward(dev, ws)
        gave_up, epoch = libwkv.workspace_query(ws)
        assert gave_up == 0 and epoch == 2 * (i + 1), (gave_up, epoch)


def test_bf16_row_pairs_match_two_byte_lanes():
    """Even C with 4-byte aligned arrays moves bfloat16 rows in pairs; a gk that is only
    2-byte aligned takes 2-byte lanes.  The arithmetic per channel is the same, so the
    gradients must agree bit for bit."""
    inp = grad_inputs(2, 700, 192, seed=31, dtype="bf16", k_std=1.5)
    dev = to_device(inp)
    pair = libwkv.wkv_backward(dev["w"], dev["u"], dev["k"], dev["v"], dev["gy"])
    buf = torch.empty(dev["k"].numel() + 1, dtype=torch.bfloat16, device="cuda")
    gk_odd = buf[1:].view(dev["k"].shape)
    assert gk_odd.data_ptr() % 4 == 2
    lanes = libwkv.wkv_backward(dev["w"], dev["u"], dev["k"], dev["v"], dev["gy"], gk=gk_odd)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, pair, lanes):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("dtype,B,T,C", [("f32", 2, 1000, 130), ("f32", 1, 100, 64), ("bf16", 2, 700, 192),
                                         ("bf16", 1, 300, 67)])
def test_saved_states_give_the_same_gradients(dtype, B, T, C):
    """wkv_forward_save gives wkv_forward's chunked y; wkv_backward_saved gives wkv_backward's
    gradients bit for bit; the saved pair needs one scan per call on its workspace."""
    inp = grad_inputs(B, T, C, seed=41 + T, dtype=dtype, k_std=1.5)
    dev = to_device(inp)
    y_ref = libwkv.wkv_forward(dev["w"], dev["u"], dev["k"], dev["v"], algo="chunked")
    y, saved = libwkv.wkv_forward_save(dev["w"], dev["u"], dev["k"], dev["v"])
    ref = libwkv.wkv_backward(dev["w"], dev["u"], dev["k"], dev["v"], dev["gy"])
    ws = libwkv.new_backward_workspace(B, T, C, dev["k"].dtype)
    got = libwkv.wkv_backward(dev["w"], dev["u"], dev["k"], dev["v"], dev["gy"], saved=saved, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    for name, a, b in zip(NAMES, got, ref):
        assert torch.equal(a, b), name
    gave_up, epoch = libwkv.workspace_query(ws)
    assert gave_up == 0 and epoch == 1
