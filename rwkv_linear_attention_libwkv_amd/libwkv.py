"""Python binding of libwkv (ctypes): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI declared
in include/libwkv.h.  torch tensors serve as device memory and
``torch.cuda.current_stream()`` as the stream; nothing here computes WKV, and
importing this module fails loudly when libwkv.so has not been built.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libwkv.so")

WKV_OK, WKV_EINVAL, WKV_EDTYPE, WKV_EWORKSPACE, WKV_EHIP = range(5)
WKV_F32, WKV_BF16 = 0, 1
ALGOS = {"auto": 0, "seq": 1, "chunked": 2}
P_EMPTY = -1.0e38

#: every function include/libwkv.h declares
EXPORTS = (
    "wkv_forward_workspace_bytes",
    "wkv_forward_workspace_init",
    "wkv_forward_workspace_query",
    "wkv_workspace_force_give_up",
    "wkv_forward",
    "wkv_forward_noalloc",
    "wkv_forward_ex",
    "wkv_forward_state",
    "wkv_step",
    "wkv_backward_workspace_bytes",
    "wkv_backward",
    "wkv_saved_states_bytes",
    "wkv_forward_save",
    "wkv_backward_saved",
    "wkv_token_shift",
    "wkv_token_shift_backward_workspace_bytes",
    "wkv_token_shift_backward",
    "wkv_forward_gated",
    "wkv_backward_gated",
    "wkv_linear_attention_workspace_bytes",
    "wkv_linear_attention",
    "wkv_linear_attention_ex",
    "wkv_status_string",
)


class WkvError(RuntimeError):
    """A libwkv call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m rwkv_linear_attention_libwkv_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation"
        )
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.wkv_forward_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i64]
    lib.wkv_forward_workspace_bytes.restype = sz
    lib.wkv_forward_workspace_init.argtypes = [vp, sz, vp]
    lib.wkv_forward_workspace_init.restype = i32
    lib.wkv_forward_workspace_query.argtypes = [vp, sz, ctypes.POINTER(ctypes.c_uint32),
                                                ctypes.POINTER(ctypes.c_uint32), vp]
    lib.wkv_forward_workspace_query.restype = i32
    lib.wkv_workspace_force_give_up.argtypes = [vp, sz, ctypes.c_uint32, vp]
    lib.wkv_workspace_force_give_up.restype = i32
    lib.wkv_forward.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.wkv_forward.restype = i32
    lib.wkv_forward_noalloc.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.wkv_forward_noalloc.restype = i32
    lib.wkv_forward_ex.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, i32, i64, vp]
    lib.wkv_forward_ex.restype = i32
    lib.wkv_forward_state.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp, vp, sz, i32, i64, vp]
    lib.wkv_forward_state.restype = i32
    lib.wkv_step.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.wkv_step.restype = i32
    lib.wkv_backward_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.wkv_backward_workspace_bytes.restype = sz
    lib.wkv_backward.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.wkv_backward.restype = i32
    lib.wkv_saved_states_bytes.argtypes = [i64, i64, i64]
    lib.wkv_saved_states_bytes.restype = sz
    lib.wkv_forward_save.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.wkv_forward_save.restype = i32
    lib.wkv_backward_saved.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, sz, vp]
    lib.wkv_backward_saved.restype = i32
    lib.wkv_token_shift.argtypes = [i64, i64, i64, i32, vp, vp, vp, i64, vp, vp]
    lib.wkv_token_shift.restype = i32
    lib.wkv_token_shift_backward_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.wkv_token_shift_backward_workspace_bytes.restype = sz
    lib.wkv_token_shift_backward.argtypes = [i64, i64, i64, i32, vp, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.wkv_token_shift_backward.restype = i32
    lib.wkv_forward_gated.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.wkv_forward_gated.restype = i32
    lib.wkv_backward_gated.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp,
                                       sz, vp]
    lib.wkv_backward_gated.restype = i32
    lib.wkv_linear_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.wkv_linear_attention_workspace_bytes.restype = sz
    lib.wkv_linear_attention.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.wkv_linear_attention.restype = i32
    lib.wkv_linear_attention_ex.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp, i32, vp, sz, i32, vp]
    lib.wkv_linear_attention_ex.restype = i32
    lib.wkv_status_string.argtypes = [i32]
    lib.wkv_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def wkv_status_string(status: int) -> str:
    return lib.wkv_status_string(int(status)).decode()


status_string = wkv_status_string


def _check(status: int, where: str):
    if status != WKV_OK:
        raise WkvError(status, where)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return WKV_F32
    if t == torch.bfloat16:
        return WKV_BF16
    raise TypeError(f"k, v must be float32 or bfloat16, got {t}")


def _ptr(t):
    # the argtypes declare c_void_p, so ctypes converts the integer address itself
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with ``stream`` (when given) as torch's current stream, so that every
    tensor it allocates (outputs, workspaces) comes from that stream's pool and is
    zero-filled on it, ordered before the launch; the caching allocator then also
    returns temporaries to that stream, after the launch that used them."""

    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)

    return wrapper


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _gpu_args(**tensors):
    """Every given tensor (None entries skipped) is a contiguous tensor on the current GPU.  The
    kernels take raw device pointers: a host or other-device pointer would fault the GPU, so it
    is refused here."""
    cur = -1
    for name, t in tensors.items():
        if t is None:
            continue
        _need(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a GPU tensor")
        if cur < 0:
            cur = torch.cuda.current_device()
        _need(t.get_device() == cur, f"{name} is on {t.device}, the launch goes to cuda:{cur}")
        _need(t.is_contiguous(), f"{name} must be contiguous")


def _same(name, t, shape, dtype):
    """A caller's output tensor has the shape and dtype the call writes."""
    _need(tuple(t.shape) == tuple(shape) and t.dtype == dtype, f"{name} must be {dtype} of shape {tuple(shape)}")


def wkv_forward_workspace_bytes(B: int, T: int, C: int, dtype=torch.float32, algo: str = "auto",
                                chunk_len: int = 0) -> int:
    n = lib.wkv_forward_workspace_bytes(B, T, C, _dtype_code(dtype), ALGOS[algo], chunk_len)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid arguments for the workspace query")
    return int(n)


@_on_stream
def wkv_forward_workspace_init(workspace, stream=None):
    """Zero-fill a forward workspace (needed once, before its first use)."""
    _gpu_args(workspace=workspace)
    _check(lib.wkv_forward_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)), "wkv_forward_workspace_init")
    return workspace


@_on_stream
def new_workspace(B: int, T: int, C: int, dtype=torch.float32, algo: str = "auto", chunk_len: int = 0,
                  device="cuda", stream=None):
    """A ready (zero-filled) workspace for these sizes, or None if none is needed.  It is
    allocated from, and zero-filled on, ``stream`` (default: torch's current stream)."""
    need = wkv_forward_workspace_bytes(B, T, C, dtype, algo, chunk_len)
    if not need:
        return None
    ws = torch.empty((need + 3) // 4 * 4, dtype=torch.uint8, device=device)
    return wkv_forward_workspace_init(ws, stream=stream)


@_on_stream
def wkv_forward(w, u, k, v, *, algo: str = "auto", chunk_len: int = 0, y=None, workspace=None,
                state=None, return_state: bool = False, state_out=None, stream=None):
    """y = WKV(w, u, k, v) for k, v of shape [B, T, C] (float32 or bfloat16, on the GPU).

    Calls wkv_forward_ex, or wkv_forward_state when a state goes in or out.

    state: optional (a, b, p) float32 tensors of shape [B, C] to start from.
    return_state: also return the state after the last token as (a, b, p)
    (written into ``state_out`` when given; may be the ``state`` tensors).
    """
    _need(k.dim() == 3 and v.shape == k.shape, "k and v must both be [B, T, C]")
    _need(k.is_cuda and v.is_cuda and w.is_cuda and u.is_cuda, "all tensors must be on the GPU")
    _need(k.dtype == v.dtype, "k and v must share a dtype")
    _need(k.is_contiguous() and v.is_contiguous(), "k and v must be contiguous")
    B, T, C = k.shape
    _need(w.dtype == torch.float32 and u.dtype == torch.float32, "w and u must be float32")
    _need(w.numel() == C and u.numel() == C and w.is_contiguous() and u.is_contiguous(),
          "w and u must be contiguous with C entries")
    dt = _dtype_code(k.dtype)
    if y is None:
        y = torch.empty_like(k)
    _need(y.shape == k.shape and y.dtype == k.dtype and y.is_contiguous(), "bad y")
    need = wkv_forward_workspace_bytes(B, T, C, k.dtype, algo, chunk_len)
    if need and workspace is None:
        workspace = new_workspace(B, T, C, k.dtype, algo, chunk_len, device=k.device, stream=stream)
    _gpu_args(w=w, u=u, k=k, v=v, y=y, workspace=workspace)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _stream(stream)
    if state is None and not return_state:
        _check(lib.wkv_forward_ex(B, T, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                  ws_ptr, ws_bytes, ALGOS[algo], chunk_len, st), "wkv_forward_ex")
        return y
    sin = (None, None, None)
    if state is not None:
        sin = tuple(state)
        for t in sin:
            _need(t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and t.numel() == B * C,
                  "state tensors must be contiguous float32 with B*C entries")
    sout = (None, None, None)
    if return_state:
        sout = tuple(state_out) if state_out is not None else tuple(
            torch.empty((B, C), dtype=torch.float32, device=k.device) for _ in range(3))
        for t in sout:
            _need(t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and t.numel() == B * C,
                  "state tensors must be contiguous float32 with B*C entries")
    _gpu_args(state_a=sin[0], state_b=sin[1], state_p=sin[2], out_a=sout[0], out_b=sout[1], out_p=sout[2])
    _check(lib.wkv_forward_state(B, T, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                 *(_ptr(t) for t in sin), *(_ptr(t) for t in sout),
                                 ws_ptr, ws_bytes, ALGOS[algo], chunk_len, st), "wkv_forward_state")
    return (y, sout) if return_state else y


@_on_stream
def wkv_forward_noalloc(w, u, k, v, *, y=None, stream=None):
    """y = WKV(w, u, k, v) through wkv_forward_noalloc: the library's static device array serves
    as the workspace (nothing allocated by the call; y is allocated here when not given)."""
    _need(k.dim() == 3 and v.shape == k.shape and k.dtype == v.dtype, "k and v must be [B, T, C] of one dtype")
    _need(k.is_cuda and k.is_contiguous() and v.is_contiguous(), "k and v must be contiguous GPU tensors")
    B, T, C = k.shape
    _need(w.dtype == torch.float32 and u.dtype == torch.float32 and w.numel() == C and u.numel() == C,
          "w and u must be float32 with C entries")
    if y is None:
        y = torch.empty_like(k)
    _need(y.shape == k.shape and y.dtype == k.dtype and y.is_contiguous(), "bad y")
    _gpu_args(w=w, u=u, k=k, v=v, y=y)
    _check(lib.wkv_forward_noalloc(B, T, C, _dtype_code(k.dtype), _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                   _stream(stream)), "wkv_forward_noalloc")
    return y


@_on_stream
def wkv_step(w, u, k, v, a, b, p, *, y=None, stream=None):
    """One decoding step for k, v of shape [N, G, C]; (a, b, p) [N, G, C] float32 updated in place.

    w, u: float32 [G, C].  Returns y (dtype of k).
    """
    _need(k.dim() == 3 and v.shape == k.shape, "k and v must both be [N, G, C]")
    N, G, C = k.shape
    _need(k.dtype == v.dtype and k.is_contiguous() and v.is_contiguous(), "bad k or v")
    for t in (a, b, p):
        _need(t.shape == k.shape and t.dtype == torch.float32 and t.is_contiguous() and t.is_cuda,
              "a, b, p must be contiguous float32 [N, G, C]")
    _need(w.dtype == torch.float32 and u.dtype == torch.float32, "w and u must be float32")
    _need(w.numel() == G * C and u.numel() == G * C and w.is_contiguous() and u.is_contiguous(),
          "w and u must be contiguous [G, C]")
    if y is None:
        y = torch.empty_like(k)
    _need(y.shape == k.shape and y.dtype == k.dtype and y.is_contiguous(), "bad y")
    _gpu_args(w=w, u=u, k=k, v=v, a=a, b=b, p=p, y=y)
    _check(lib.wkv_step(N, G, C, _dtype_code(k.dtype), _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                        _ptr(a), _ptr(b), _ptr(p), _ptr(y), _stream(stream)), "wkv_step")
    return y


def wkv_backward_workspace_bytes(B: int, T: int, C: int, dtype=torch.float32) -> int:
    n = lib.wkv_backward_workspace_bytes(B, T, C, _dtype_code(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid arguments for the workspace query")
    return int(n)


@_on_stream
def new_backward_workspace(B: int, T: int, C: int, dtype=torch.float32, device="cuda", stream=None):
    """A ready (zero-filled) backward workspace for these sizes, or None if none is needed
    (allocated from, and zero-filled on, ``stream``)."""
    need = wkv_backward_workspace_bytes(B, T, C, dtype)
    if not need:
        return None
    ws = torch.empty((need + 3) // 4 * 4, dtype=torch.uint8, device=device)
    return wkv_forward_workspace_init(ws, stream=stream)


def wkv_saved_states_bytes(B: int, T: int, C: int) -> int:
    n = lib.wkv_saved_states_bytes(B, T, C)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for the saved-state query")
    return int(n)


@_on_stream
def wkv_forward_save(w, u, k, v, *, y=None, saved=None, workspace=None, stream=None):
    """y = WKV(w, u, k, v) plus the states wkv_backward_saved needs: returns (y, saved).

    ``saved`` is an opaque uint8 device tensor of wkv_saved_states_bytes(B, T, C) bytes.
    """
    _need(k.dim() == 3 and v.shape == k.shape and k.dtype == v.dtype, "k and v must be [B, T, C] of one dtype")
    _need(k.is_contiguous() and v.is_contiguous() and k.is_cuda, "k and v must be contiguous GPU tensors")
    B, T, C = k.shape
    _need(w.numel() == C and u.numel() == C and w.dtype == torch.float32 and u.dtype == torch.float32,
          "w and u must be float32 with C entries")
    y = torch.empty_like(k) if y is None else y
    _need(y.shape == k.shape and y.dtype == k.dtype and y.is_contiguous(), "bad y")
    nbytes = wkv_saved_states_bytes(B, T, C)
    if saved is None:
        saved = torch.empty(max(4, nbytes), dtype=torch.uint8, device=k.device)
    _need(saved.is_cuda and saved.is_contiguous(), "bad saved buffer")
    if workspace is None:
        workspace = new_workspace(B, T, C, k.dtype, "chunked", 0, device=k.device, stream=stream)
    _gpu_args(w=w, u=u, k=k, v=v, y=y, saved=saved, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.wkv_forward_save(B, T, C, _dtype_code(k.dtype), _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                _ptr(saved), saved.numel() * saved.element_size(), _ptr(workspace), ws_bytes,
                                _stream(stream)), "wkv_forward_save")
    return y, saved


@_on_stream
def wkv_backward(w, u, k, v, gy, *, saved=None, gk=None, gv=None, gw=None, gu=None, workspace=None,
                 stream=None):
    """Gradients of sum(gy * WKV(w, u, k, v)): returns (gw, gu, gk, gv).

    k, v, gy: [B, T, C] (float32 or bfloat16, on the GPU); gk, gv have their dtype;
    gw, gu are float32 [B, C] per-lane gradients (sum over B for the [C] parameters).
    With ``saved`` (from wkv_forward_save) calls wkv_backward_saved, else wkv_backward.
    """
    _need(k.dim() == 3 and v.shape == k.shape and gy.shape == k.shape, "k, v and gy must be [B, T, C]")
    _need(k.is_cuda and v.is_cuda and gy.is_cuda and w.is_cuda and u.is_cuda, "all tensors must be on the GPU")
    _need(k.dtype == v.dtype == gy.dtype, "k, v and gy must share a dtype")
    _need(k.is_contiguous() and v.is_contiguous() and gy.is_contiguous(), "k, v and gy must be contiguous")
    B, T, C = k.shape
    _need(w.dtype == torch.float32 and u.dtype == torch.float32, "w and u must be float32")
    _need(w.numel() == C and u.numel() == C and w.is_contiguous() and u.is_contiguous(),
          "w and u must be contiguous with C entries")
    gk = torch.empty_like(k) if gk is None else gk
    gv = torch.empty_like(k) if gv is None else gv
    for t in (gk, gv):
        _need(t.shape == k.shape and t.dtype == k.dtype and t.is_contiguous(), "bad gk or gv")
    gw = torch.empty((B, C), dtype=torch.float32, device=k.device) if gw is None else gw
    gu = torch.empty((B, C), dtype=torch.float32, device=k.device) if gu is None else gu
    for t in (gw, gu):
        _need(t.numel() == B * C and t.dtype == torch.float32 and t.is_contiguous(), "bad gw or gu")
    if workspace is None:
        workspace = new_backward_workspace(B, T, C, k.dtype, device=k.device, stream=stream)
    _gpu_args(w=w, u=u, k=k, v=v, gy=gy, gk=gk, gv=gv, gw=gw, gu=gu, saved=saved, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if saved is None:
        _check(lib.wkv_backward(B, T, C, _dtype_code(k.dtype), _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(gy),
                                _ptr(gk), _ptr(gv), _ptr(gw), _ptr(gu), _ptr(workspace), ws_bytes,
                                _stream(stream)), "wkv_backward")
    else:
        _need(saved.is_cuda and saved.is_contiguous(), "bad saved buffer")
        _check(lib.wkv_backward_saved(B, T, C, _dtype_code(k.dtype), _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                      _ptr(gy), _ptr(saved), saved.numel() * saved.element_size(), _ptr(gk),
                                      _ptr(gv), _ptr(gw), _ptr(gu), _ptr(workspace), ws_bytes, _stream(stream)),
               "wkv_backward_saved")
    return gw, gu, gk, gv


@_on_stream
def wkv_token_shift(x, mu, *, x_prev=None, out=None, stream=None):
    """out[m] = mu[m] * x_t + (1 - mu[m]) * x_{t-1} for x [B, T, C], mu [M, C] float32; returns [M, B, T, C]."""
    _need(x.dim() == 3 and x.is_cuda and x.is_contiguous(), "x must be a contiguous [B, T, C] GPU tensor")
    B, T, C = x.shape
    _need(mu.dim() == 2 and mu.shape[1] == C and mu.dtype == torch.float32 and mu.is_contiguous(),
          "mu must be contiguous float32 [M, C]")
    M = mu.shape[0]
    if x_prev is not None:
        _need(x_prev.shape == (B, C) and x_prev.dtype == x.dtype and x_prev.is_contiguous(), "bad x_prev")
    out = torch.empty((M, B, T, C), dtype=x.dtype, device=x.device) if out is None else out
    _need(out.shape == (M, B, T, C) and out.dtype == x.dtype and out.is_contiguous(), "bad out")
    _gpu_args(x=x, mu=mu, x_prev=x_prev, out=out)
    _check(lib.wkv_token_shift(B, T, C, _dtype_code(x.dtype), _ptr(x), _ptr(x_prev), _ptr(mu), M, _ptr(out),
                               _stream(stream)), "wkv_token_shift")
    return out


@_on_stream
def wkv_token_shift_backward(x, mu, g, *, x_prev=None, want_gprev=True, gx=None, gmu=None, gprev=None,
                             workspace=None, stream=None):
    """Gradients of sum(g * wkv_token_shift(x, mu, x_prev)) for g [M, B, T, C]: returns
    (gx [B, T, C] dtype, gmu [M, B, C] float32 per lane, gprev [B, C] dtype or None)."""
    _need(x.dim() == 3 and x.is_cuda and x.is_contiguous(), "x must be a contiguous [B, T, C] GPU tensor")
    B, T, C = x.shape
    _need(mu.dim() == 2 and mu.shape[1] == C and mu.dtype == torch.float32 and mu.is_contiguous(),
          "mu must be contiguous float32 [M, C]")
    M = mu.shape[0]
    _need(g.shape == (M, B, T, C) and g.dtype == x.dtype and g.is_contiguous(), "g must be [M, B, T, C] of x's dtype")
    if x_prev is not None:
        _need(x_prev.shape == (B, C) and x_prev.dtype == x.dtype and x_prev.is_contiguous(), "bad x_prev")
    gx = torch.empty_like(x) if gx is None else gx
    gmu = torch.empty((M, B, C), dtype=torch.float32, device=x.device) if gmu is None else gmu
    if want_gprev and gprev is None:
        gprev = torch.empty((B, C), dtype=x.dtype, device=x.device)
    _same("gx", gx, (B, T, C), x.dtype)
    _same("gmu", gmu, (M, B, C), torch.float32)
    if gprev is not None:
        _same("gprev", gprev, (B, C), x.dtype)
    need = lib.wkv_token_shift_backward_workspace_bytes(B, T, C, M)
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for the token shift backward")
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _gpu_args(x=x, mu=mu, g=g, x_prev=x_prev, gx=gx, gmu=gmu, gprev=gprev, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.wkv_token_shift_backward(B, T, C, _dtype_code(x.dtype), _ptr(x), _ptr(x_prev), _ptr(mu), M, _ptr(g),
                                        _ptr(gx), _ptr(gmu), _ptr(gprev), _ptr(workspace), ws_bytes, _stream(stream)),
           "wkv_token_shift_backward")
    return gx, gmu, gprev


@_on_stream
def wkv_forward_gated(w, u, k, v, r, *, z=None, saved=None, workspace=None, stream=None):
    """z = sigmoid(r) * WKV(w, u, k, v).  With ``saved`` (a uint8 device tensor of
    wkv_saved_states_bytes bytes) also keeps the states for wkv_backward_gated."""
    _need(k.dim() == 3 and v.shape == k.shape and r.shape == k.shape, "k, v and r must be [B, T, C]")
    _need(k.dtype == v.dtype == r.dtype, "k, v and r must share a dtype")
    _need(k.is_contiguous() and v.is_contiguous() and r.is_contiguous() and k.is_cuda, "bad k, v or r")
    B, T, C = k.shape
    _need(w.numel() == C and u.numel() == C and w.dtype == torch.float32 and u.dtype == torch.float32,
          "w and u must be float32 with C entries")
    z = torch.empty_like(k) if z is None else z
    _need(z.shape == k.shape and z.dtype == k.dtype and z.is_contiguous(), "bad z")
    algo = "chunked" if saved is not None else "auto"
    if workspace is None:
        workspace = new_workspace(B, T, C, k.dtype, algo, 0, device=k.device, stream=stream)
    _gpu_args(w=w, u=u, k=k, v=v, r=r, z=z, saved=saved, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sb = 0 if saved is None else saved.numel() * saved.element_size()
    _check(lib.wkv_forward_gated(B, T, C, _dtype_code(k.dtype), _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(z),
                                 _ptr(saved), sb, _ptr(workspace), ws_bytes, _stream(stream)), "wkv_forward_gated")
    return z


@_on_stream
def wkv_backward_gated(w, u, k, v, r, gz, *, saved=None, gk=None, gv=None, gr=None, gw=None, gu=None,
                       workspace=None, stream=None):
    """Gradients of sum(gz * sigmoid(r) * WKV(w, u, k, v)): returns (gw, gu, gk, gv, gr)."""
    _need(k.dim() == 3 and all(t.shape == k.shape for t in (v, r, gz)), "k, v, r and gz must be [B, T, C]")
    _need(all(t.dtype == k.dtype and t.is_contiguous() and t.is_cuda for t in (v, r, gz)), "bad v, r or gz")
    B, T, C = k.shape
    _need(w.dtype == torch.float32 and u.dtype == torch.float32 and w.numel() == C and u.numel() == C,
          "w and u must be float32 with C entries")
    gk = torch.empty_like(k) if gk is None else gk
    gv = torch.empty_like(k) if gv is None else gv
    gr = torch.empty_like(k) if gr is None else gr
    gw = torch.empty((B, C), dtype=torch.float32, device=k.device) if gw is None else gw
    gu = torch.empty((B, C), dtype=torch.float32, device=k.device) if gu is None else gu
    for name, t in (("gk", gk), ("gv", gv), ("gr", gr)):
        _same(name, t, k.shape, k.dtype)
    for name, t in (("gw", gw), ("gu", gu)):
        _need(t.numel() == B * C and t.dtype == torch.float32, f"{name} must be float32 with B*C entries")
    if workspace is None:
        workspace = new_backward_workspace(B, T, C, k.dtype, device=k.device, stream=stream)
    _gpu_args(w=w, u=u, k=k, v=v, r=r, gz=gz, gk=gk, gv=gv, gr=gr, gw=gw, gu=gu, saved=saved,
              workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sb = 0 if saved is None else saved.numel() * saved.element_size()
    _check(lib.wkv_backward_gated(B, T, C, _dtype_code(k.dtype), _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                  _ptr(gz), _ptr(saved), sb, _ptr(gk), _ptr(gv), _ptr(gr), _ptr(gw), _ptr(gu),
                                  _ptr(workspace), ws_bytes, _stream(stream)), "wkv_backward_gated")
    return gw, gu, gk, gv, gr


@_on_stream
def new_la_workspace(BH: int, N: int, D: int, M: int, dtype=torch.float32, device="cuda", stream=None):
    """A ready (zero-filled) linear-attention workspace for these sizes, or None if none is needed
    (allocated from, and zero-filled on, ``stream``).  It may serve any number of later calls of
    these sizes (one at a time)."""
    need = lib.wkv_linear_attention_workspace_bytes(BH, N, D, M, _dtype_code(dtype))
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported linear attention shape (D and M each 32 or 64)")
    if not need:
        return None
    ws = torch.empty((need + 3) // 4 * 4, dtype=torch.uint8, device=device)
    return wkv_forward_workspace_init(ws, stream=stream)


LA_ALGOS = {"auto": 0, "three": 1, "one": 2}


@_on_stream
def linear_attention(q, k, v, *, feature_map=True, out=None, workspace=None, algo: str = "auto", stream=None):
    """Causal linear attention for q, k [BH, N, D] and v [BH, N, M] (float32 or bfloat16).
    algo: "one" (one launch, look-backs), "three" (aggregates, scan, outputs) or "auto"."""
    _need(q.dim() == 3 and k.shape == q.shape and v.dim() == 3 and v.shape[:2] == q.shape[:2],
          "q, k must be [BH, N, D] and v [BH, N, M]")
    _need(q.dtype == k.dtype == v.dtype and all(t.is_cuda and t.is_contiguous() for t in (q, k, v)),
          "q, k, v must be contiguous GPU tensors of one dtype")
    BH, N, D = q.shape
    M = v.shape[2]
    out = torch.empty_like(v) if out is None else out
    _need(out.shape == v.shape and out.dtype == v.dtype and out.is_contiguous(), "bad out")
    need = lib.wkv_linear_attention_workspace_bytes(BH, N, D, M, _dtype_code(q.dtype))
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported linear attention shape (D and M each 32 or 64)")
    if workspace is None and need:
        workspace = new_la_workspace(BH, N, D, M, q.dtype, device=q.device, stream=stream)
    _gpu_args(q=q, k=k, v=v, out=out, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.wkv_linear_attention_ex(BH, N, D, M, _dtype_code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                       1 if feature_map else 0, _ptr(workspace), ws_bytes, LA_ALGOS[algo],
                                       _stream(stream)),
           "wkv_linear_attention_ex")
    return out


def empty_state(shape, device="cuda"):
    """(a, b, p) float32 tensors of the empty state (a = b = 0, p = P_EMPTY)."""
    a = torch.zeros(shape, dtype=torch.float32, device=device)
    b = torch.zeros(shape, dtype=torch.float32, device=device)
    p = torch.full(shape, P_EMPTY, dtype=torch.float32, device=device)
    return a, b, p


def workspace_query(workspace, stream=None):
    """(gave_up, epoch) of a forward workspace; synchronises the stream first."""
    _gpu_args(workspace=workspace)
    g, e = ctypes.c_uint32(0), ctypes.c_uint32(0)
    _check(lib.wkv_forward_workspace_query(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                           ctypes.byref(g), ctypes.byref(e), _stream(stream)),
           "wkv_forward_workspace_query")
    return int(g.value), int(e.value)


def force_give_up(workspace, launches: int = 1, stream=None):
    """Test hook: the next ``launches`` chained-scan launches on ``workspace`` take the give-up
    path in every tile (entering states rebuilt without waiting); see wkv_workspace_force_give_up."""
    _gpu_args(workspace=workspace)
    _check(lib.wkv_workspace_force_give_up(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                           int(launches), _stream(stream)), "wkv_workspace_force_give_up")


def lookback_error(workspace, stream=None) -> int:
    """Non-zero if the last chunked call on ``workspace`` had a tile give up waiting (its outputs
    are still valid: such tiles rebuild their state without waiting)."""
    return workspace_query(workspace, stream)[0]


def workspace_epoch(workspace, stream=None) -> int:
    """Launch counter kept in a chunked workspace."""
    return workspace_query(workspace, stream)[1]


# short aliases
forward = wkv_forward
step = wkv_step
backward = wkv_backward
forward_save = wkv_forward_save
token_shift = wkv_token_shift
token_shift_backward = wkv_token_shift_backward
forward_gated = wkv_forward_gated
backward_gated = wkv_backward_gated
workspace_bytes = wkv_forward_workspace_bytes
