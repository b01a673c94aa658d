"""wkv_forward_noalloc (the static device array as workspace) against wkv_forward with a
workspace: the same kernels, so the outputs must agree bit for bit, and both meet the forward's
gate against the float64 oracle.  Two calls in a row, the second smaller, through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import scaled_error, wkv_recurrent
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TOL, host, to_device

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20


def call_noalloc(dev, y):
    B, T, C = dev["k"].shape
    st = torch.cuda.current_stream().cuda_stream
    return libwkv.lib.wkv_forward_noalloc(B, T, C, libwkv._dtype_code(dev["k"].dtype),
                                          ctypes.c_void_p(dev["w"].data_ptr()), ctypes.c_void_p(dev["u"].data_ptr()),
                                          ctypes.c_void_p(dev["k"].data_ptr()), ctypes.c_void_p(dev["v"].data_ptr()),
                                          ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(st))


@pytest.mark.parametrize("first,second", [
    (("f32", 2, 5000, 256), ("f32", 1, 3000, 130)),
    (("bf16", 1, 20000, 512), ("bf16", 2, 4100, 128)),
])
def test_noalloc_matches_forward(first, second):
    for dtype, B, T, C in (first, second):
        assert libwkv.wkv_forward_workspace_bytes(B, T, C, torch.float32 if dtype == "f32" else torch.bfloat16) > 0
        inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, dtype=dtype, seed=T + C, k_std=1.5))
        dev = to_device(inp)
        y_na = torch.full_like(dev["k"], 3.0)
        assert call_noalloc(dev, y_na) == libwkv.WKV_OK
        y_ws = libwkv.wkv_forward(dev["w"], dev["u"], dev["k"], dev["v"])
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), (dtype, B, T, C)
        y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
        err = scaled_error(host(y_na), y_ref, s_ref)
        print(f"  noalloc {dtype} B={B} T={T} C={C}: {err:.2e}", flush=True)
        assert err <= TOL[dtype], err


def test_noalloc_rejects_problems_beyond_the_array():
    """More than 32 MiB of workspace and more batch rows than the sequential kernel's grid holds:
    WKV_EWORKSPACE before any launch (dummy pointers)."""
    B, T, C = 65536, 4096, 64
    need = libwkv.wkv_forward_workspace_bytes(B, T, C, torch.bfloat16)
    assert need > SCRATCH_BYTES
    p = ctypes.c_void_p(0x1000)
    assert libwkv.lib.wkv_forward_noalloc(B, T, C, libwkv.WKV_BF16, p, p, p, p, p, None) == libwkv.WKV_EWORKSPACE


def test_noalloc_beyond_the_array_runs_sequentially():
    """More than 32 MiB of workspace with B <= 65535: the sequential algorithm, bit for bit what
    wkv_forward gives with algo="seq", and within the tolerance of the oracle on sampled rows."""
    B, T, C = 512, 512, 768
    assert libwkv.wkv_forward_workspace_bytes(B, T, C, torch.float32) > SCRATCH_BYTES
    inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, seed=12))
    dev = to_device(inp)
    y = torch.empty_like(dev["k"])
    assert call_noalloc(dev, y) == libwkv.WKV_OK
    y_seq = libwkv.wkv_forward(dev["w"], dev["u"], dev["k"], dev["v"], algo="seq")
    torch.cuda.synchronize()
    assert torch.equal(y, y_seq)
    rows = [0, 1, 255, 511]
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"][rows], inp["v"][rows], return_scale=True)
    assert scaled_error(host(y[rows]), y_ref, s_ref) <= TOL["f32"]


def test_noalloc_sequential_and_empty():
    """Problems that need no workspace (many lanes: the sequential kernel; empty sizes)."""
    inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=1, T=40, C=96, seed=2))
    dev = to_device(inp)
    y = torch.empty_like(dev["k"])
    assert call_noalloc(dev, y) == libwkv.WKV_OK
    torch.cuda.synchronize()
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    assert scaled_error(host(y), y_ref, s_ref) <= TOL["f32"]
    e = torch.empty((1, 0, 96), device="cuda")
    assert libwkv.lib.wkv_forward_noalloc(1, 0, 96, libwkv.WKV_F32, None, None, None, None, None, None) == libwkv.WKV_OK
    del e
