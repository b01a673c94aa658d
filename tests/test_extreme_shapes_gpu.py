"""Forward and backward at the edges of the shapes the library accepts, against the oracle.

Wide rows: C above a million channels (1 M + 66 float32, 1 M + 34 bf16 row pairs), so that a
wave's row window spans 64 rows of 4 MB or 2 MB and the last channel group is ragged; checked on
sampled channels, the first and the last included.  A long sequence: one sequence of 2^18 + 37
tokens over 66 channels, so that one channel group chains 1025 tiles of 256 (or 513 of 512) and
the last is ragged; every output checked.  Gates as everywhere: forward 2e-5 (float32) / 1e-2
(bf16), gradients 5e-5 (float32).
"""
import numpy as np
import pytest
import torch

from oracle import scaled_error, wkv_backward_recurrent, wkv_recurrent
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TOL, host, run_forward, to_device
from tests.test_backward_gpu import TOL_F32, grad_error

pytestmark = pytest.mark.gpu


def sampled_channels(C, n=192, seed=0):
    cs = np.random.default_rng(seed).choice(C, n, replace=False)
    return np.unique(np.concatenate([cs, [0, 1, 63, 64, C - 2, C - 1]]))


@pytest.mark.parametrize("dtype,C", [("f32", (1 << 20) + 66), ("bf16", (1 << 20) + 34)])
def test_wide_rows_forward(dtype, C):
    spec = workloads.FWD_SMALL.with_(B=1, T=130, C=C, dtype=dtype, seed=41)
    inp = workloads.forward_inputs(spec)
    cs = sampled_channels(C)
    ref, scale = wkv_recurrent(inp["w"][cs], inp["u"][cs], inp["k"][:, :, cs], inp["v"][:, :, cs],
                               return_scale=True)
    dev = to_device(inp)
    del inp
    for algo, cl in (("auto", 0), ("seq", 0), ("chunked", 128)):  # auto: the chunked scan at its default tile
        y = run_forward(dev, algo, cl)
        err = scaled_error(host(y[:, :, torch.from_numpy(cs).cuda()]), ref, scale)
        print(f"  wide rows {dtype} C={C} {algo} {cl}: {err:.2e}", flush=True)
        assert err <= TOL[dtype], (algo, err)
        del y
        torch.cuda.empty_cache()


def test_wide_rows_backward():
    C = (1 << 20) + 66
    spec = workloads.FWD_SMALL.with_(B=1, T=130, C=C, seed=42)
    inp = workloads.backward_inputs(spec)
    cs = sampled_channels(C, seed=1)
    ref, scale = wkv_backward_recurrent(inp["w"][cs], inp["u"][cs], inp["k"][:, :, cs], inp["v"][:, :, cs],
                                        inp["gy"][:, :, cs], return_scale=True)
    dev = to_device(inp)
    gy = torch.from_numpy(inp["gy"]).cuda()
    del inp
    idx = torch.from_numpy(cs).cuda()
    gw, gu, gk, gv = libwkv.wkv_backward(dev["w"], dev["u"], dev["k"], dev["v"], gy)
    got = (host(gw[:, idx]), host(gu[:, idx]), host(gk[:, :, idx]), host(gv[:, :, idx]))
    for name, g, r, s in zip(("gw", "gu", "gk", "gv"), got, ref, scale):
        err = grad_error(g, r, s)
        print(f"  wide rows backward {name}: {err:.2e}", flush=True)
        assert err <= TOL_F32, (name, err)


def test_long_sequence_forward():
    B, T, C = 1, (1 << 18) + 37, 66
    inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, seed=43))
    ref, scale = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    dev = to_device(inp)
    for algo, cl in (("seq", 0), ("chunked", 256), ("chunked", 512)):
        err = scaled_error(host(run_forward(dev, algo, cl)), ref, scale)
        print(f"  long sequence T={T} {algo} {cl}: {err:.2e}", flush=True)
        assert err <= TOL["f32"], (algo, cl, err)
