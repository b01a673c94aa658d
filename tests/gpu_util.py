"""Helpers shared by the GPU tests: move seeded inputs to the device, run libwkv, compare."""
import numpy as np
import torch

from rwkv_linear_attention_libwkv_amd import libwkv

TOL = {"f32": 2e-5, "bf16": 1e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(inp):
    dt = TORCH_DT[inp["dtype"]]
    return {
        "w": torch.from_numpy(np.ascontiguousarray(inp["w"])).cuda(),
        "u": torch.from_numpy(np.ascontiguousarray(inp["u"])).cuda(),
        "k": torch.from_numpy(np.ascontiguousarray(inp["k"])).cuda().to(dt),
        "v": torch.from_numpy(np.ascontiguousarray(inp["v"])).cuda().to(dt),
    }


def run_forward(dev, algo="auto", chunk_len=0, state=None, return_state=False):
    """Run wkv_forward on device tensors; asserts the look-back never gave up."""
    k = dev["k"]
    B, T, C = k.shape
    ws = libwkv.new_workspace(B, T, C, k.dtype, algo, chunk_len, device=k.device)
    out = libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo=algo, chunk_len=chunk_len,
                             workspace=ws, state=state, return_state=return_state)
    torch.cuda.synchronize()
    if ws is not None:
        assert libwkv.lookback_error(ws) == 0, "look-back gave up waiting"
    return out


def host(t):
    return t.float().cpu().numpy().astype(np.float64)
