"""Host-side checks of the libwkv C ABI: no GPU needed.

Every argument check runs before any HIP call, so invalid calls are exercised
here with dummy pointers; nothing in this file launches a kernel.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libwkv.h")

from rwkv_linear_attention_libwkv_amd import libwkv  # noqa: E402

lib = libwkv.lib
OK, EINVAL, EDTYPE, EWS = libwkv.WKV_OK, libwkv.WKV_EINVAL, libwkv.WKV_EDTYPE, libwkv.WKV_EWORKSPACE
F32, BF16 = libwkv.WKV_F32, libwkv.WKV_BF16
P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation or is empty
NULL = None


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wkv_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function():
    declared = header_functions()
    assert set(declared) == set(libwkv.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(5):
        assert libwkv.status_string(s).startswith("WKV_")
    assert "unknown" in libwkv.status_string(99)


def fwd(B, T, C, dt=F32, w=P, u=P, k=P, v=P, y=P, ws=NULL, ws_bytes=0, algo=0, chunk=0):
    return lib.wkv_forward_ex(B, T, C, dt, w, u, k, v, y, ws, ws_bytes, algo, chunk, None)


def test_forward_argument_checks():
    assert fwd(-1, 4, 4) == EINVAL
    assert fwd(1, -4, 4) == EINVAL
    assert fwd(1, 4, -4) == EINVAL
    assert fwd(1, 4, 4, dt=7) == EDTYPE
    assert fwd(1, 4, 4, algo=9) == EINVAL
    assert fwd(1, 4, 4, chunk=100) == EINVAL
    assert fwd(1, 4, 4, k=NULL) == EINVAL
    assert fwd(1, 4, 4, y=NULL, algo=1) == EINVAL
    assert fwd(1, 1 << 31, 4) == EINVAL
    assert fwd(1 << 20, 4, 1 << 12) == EINVAL  # B*C beyond int32
    # chunked needs a workspace of the queried size
    assert fwd(2, 1000, 64, algo=2) == EWS
    need = lib.wkv_forward_workspace_bytes(2, 1000, 64, F32, 2, 0)
    assert need > 0
    assert fwd(2, 1000, 64, algo=2, ws=P, ws_bytes=need - 1) == EWS


def test_row_window_width_limit():
    """A wave addresses up to 64 rows from one buffer resource with 32-bit offsets: widths whose
    64 rows pass 2^31 - 1 bytes are refused before any launch (float32 from C = 2^23, bf16 from 2^24)."""
    assert fwd(1, 4, 1 << 23) == EINVAL
    assert fwd(1, 4, 1 << 24, dt=BF16) == EINVAL
    # the widest accepted widths still get a workspace size (queries launch nothing)
    assert lib.wkv_forward_workspace_bytes(1, 4096, (1 << 23) - 1, F32, 2, 0) > 0
    assert lib.wkv_forward_workspace_bytes(1, 4096, (1 << 24) - 1, BF16, 2, 0) > 0
    assert lib.wkv_forward_workspace_bytes(1, 4096, 1 << 23, F32, 2, 0) == ctypes.c_size_t(-1).value
    assert lib.wkv_forward_workspace_bytes(1, 4096, 1 << 24, BF16, 2, 0) == ctypes.c_size_t(-1).value
    assert lib.wkv_backward_workspace_bytes(1, 4096, 1 << 23, F32) == ctypes.c_size_t(-1).value
    assert lib.wkv_backward(1, 4, 1 << 23, F32, P, P, P, P, P, P, P, P, P, P, 1 << 20, None) == EINVAL
    assert lib.wkv_forward_gated(1, 4, 1 << 24, BF16, P, P, P, P, P, P, NULL, 0, P, 1 << 20, None) == EINVAL


def test_forward_empty_problems_are_noops():
    for B, T, C in [(0, 5, 5), (5, 0, 5), (5, 5, 0)]:
        assert fwd(B, T, C, w=NULL, u=NULL, k=NULL, v=NULL, y=NULL) == OK


def test_forward_state_pointer_checks():
    def st(sia, sib, sip, soa, sob, sop, T=4):
        return lib.wkv_forward_state(1, T, 4, F32, P, P, P, P, P, sia, sib, sip, soa, sob, sop,
                                     None, 0, 1, 0, None)
    assert st(P, NULL, NULL, NULL, NULL, NULL) == EINVAL
    assert st(NULL, NULL, NULL, P, P, NULL) == EINVAL
    # T = 0 with the same arrays in and out: nothing to do
    assert st(P, P, P, P, P, P, T=0) == OK
    # T = 0 without state out: nothing to do
    assert st(NULL, NULL, NULL, NULL, NULL, NULL, T=0) == OK


def test_workspace_query():
    q = lib.wkv_forward_workspace_bytes
    bad = ctypes.c_size_t(-1).value
    assert q(-1, 4, 4, F32, 0, 0) == bad
    assert q(1, 4, 4, 5, 0, 0) == bad
    assert q(1, 4, 4, F32, 0, 77) == bad
    assert q(1, 4, 4, F32, 3, 0) == bad
    assert q(0, 4, 4, F32, 2, 0) == 0
    assert q(8, 8192, 2048, F32, 1, 0) == 0  # the sequential walk needs none
    a = q(8, 8192, 2048, F32, 2, 0)
    assert a > 0 and a == q(8, 8192, 2048, BF16, 2, 0)
    assert q(8, 8192, 2048, F32, 2, 64) > q(8, 8192, 2048, F32, 2, 256)
    # AUTO picks the chunked scan for every T over 64, whatever the number of lanes, and the
    # sequential walk (no workspace) for T up to 64 unless B is beyond its grid (65535 rows)
    assert q(1, 65536, 5120, BF16, 0, 0) > 0
    assert q(1, 64, 64, F32, 0, 0) == 0
    assert q(8192, 64, 1024, F32, 0, 0) == 0
    assert q(8192, 65, 1024, F32, 0, 0) == q(8192, 65, 1024, F32, 2, 0) > 0
    assert q(1024, 1024, 768, BF16, 0, 0) == q(1024, 1024, 768, BF16, 2, 0) > 0
    assert q(65536, 64, 64, F32, 0, 0) == q(65536, 64, 64, F32, 2, 0) > 0


def test_workspace_diagnostics_argument_checks():
    g, e = ctypes.c_uint32(), ctypes.c_uint32()
    wq = lib.wkv_forward_workspace_query
    assert wq(NULL, 4096, ctypes.byref(g), ctypes.byref(e), None) == EINVAL
    assert wq(P, 4096, None, ctypes.byref(e), None) == EINVAL
    assert wq(P, 4096, ctypes.byref(g), None, None) == EINVAL
    # too small for the control block: rejected before any HIP call
    assert wq(P, 255, ctypes.byref(g), ctypes.byref(e), None) == EWS
    assert wq(ctypes.c_void_p(0x1004), 256, ctypes.byref(g), ctypes.byref(e), None) == EWS
    fg = lib.wkv_workspace_force_give_up
    assert fg(NULL, 4096, 1, None) == EINVAL
    assert fg(P, 255, 1, None) == EWS
    assert fg(ctypes.c_void_p(0x1004), 256, 1, None) == EWS


def test_step_argument_checks():
    def step(N, G, C, dt=BF16, ptrs=(P,) * 8):
        return lib.wkv_step(N, G, C, dt, *ptrs, None)
    assert step(-1, 2, 2) == EINVAL
    assert step(1, -2, 2) == EINVAL
    assert step(1, 2, -2) == EINVAL
    assert step(1, 2, 2, dt=3) == EDTYPE
    assert step(0, 2, 2, ptrs=(NULL,) * 8) == OK
    for i in range(8):
        ptrs = [P] * 8
        ptrs[i] = NULL
        assert step(1, 2, 2, ptrs=tuple(ptrs)) == EINVAL, i


def test_backward_argument_checks():
    def bwd(B, T, C, dt=F32, ptrs=(P,) * 9, ws=NULL, ws_bytes=0):
        return lib.wkv_backward(B, T, C, dt, *ptrs, ws, ws_bytes, None)
    assert bwd(-1, 4, 4) == EINVAL
    assert bwd(1, -4, 4) == EINVAL
    assert bwd(1, 1 << 31, 4) == EINVAL
    assert bwd(1, 4, 4, dt=5) == EDTYPE
    assert bwd(0, 4, 4, ptrs=(NULL,) * 9) == OK
    assert bwd(4, 4, 0, ptrs=(NULL,) * 9) == OK
    # every pointer operand is required for a non-empty problem (gw, gu even with T = 0)
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = NULL
        assert bwd(2, 300, 64, ptrs=tuple(ptrs), ws=P, ws_bytes=1 << 30) == EINVAL, i
    for i in (7, 8):
        ptrs = [P] * 9
        ptrs[i] = NULL
        assert bwd(2, 0, 64, ptrs=tuple(ptrs)) == EINVAL, i
    need = lib.wkv_backward_workspace_bytes(2, 300, 64, F32)
    assert need > 0
    assert bwd(2, 300, 64) == EWS
    assert bwd(2, 300, 64, ws=P, ws_bytes=need - 1) == EWS


def test_backward_workspace_query():
    q = lib.wkv_backward_workspace_bytes
    bad = ctypes.c_size_t(-1).value
    assert q(-1, 4, 4, F32) == bad
    assert q(1, 4, 4, 9) == bad
    assert q(0, 4, 4, F32) == 0 and q(4, 0, 4, F32) == 0
    a = q(8, 8192, 2048, F32)
    assert a == q(8, 8192, 2048, BF16)
    # per 128 x 64 tile: 5 tagged 8-byte words x 2 slots x 64 channels, 5 float32 planes
    # and a status word, plus the forward scan's records at its default chunk length
    elems = 8 * 8192 * 2048
    assert 0.9 * elems < a < 1.05 * elems + (1 << 20)
    assert a > lib.wkv_forward_workspace_bytes(8, 8192, 2048, F32, 2, 0)


def test_saved_state_entry_points_argument_checks():
    q = lib.wkv_saved_states_bytes
    assert q(-1, 4, 4) == ctypes.c_size_t(-1).value
    assert q(0, 4, 4) == 0 and q(4, 0, 4) == 0
    need = q(2, 300, 64)
    assert need >= 3 * 3 * 2 * 64 * 4  # three planes of ceil(300 / 128) x 128 lanes
    fs = lib.wkv_forward_save
    assert fs(2, 300, 64, F32, P, P, P, P, P, NULL, 0, P, 1 << 30, None) == EINVAL
    assert fs(2, 300, 64, F32, P, P, P, P, P, P, need - 1, P, 1 << 30, None) == EINVAL
    assert fs(2, 300, 64, 9, P, P, P, P, P, P, need, P, 1 << 30, None) == EDTYPE
    assert fs(2, 300, 64, F32, P, P, P, P, P, P, need, NULL, 0, None) == EWS
    assert fs(0, 300, 64, F32, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, None) == OK
    bs = lib.wkv_backward_saved
    wsb = lib.wkv_backward_workspace_bytes(2, 300, 64, F32)
    assert bs(2, 300, 64, F32, P, P, P, P, P, NULL, 0, P, P, P, P, P, wsb, None) == EINVAL
    assert bs(2, 300, 64, F32, P, P, P, P, P, P, need - 1, P, P, P, P, P, wsb, None) == EINVAL
    assert bs(2, 300, 64, F32, P, P, P, P, P, P, need, P, P, P, P, P, wsb - 1, None) == EWS


def test_token_shift_and_gate_argument_checks():
    ts = lib.wkv_token_shift
    assert ts(2, 8, 16, F32, P, NULL, P, 0, P, None) == EINVAL
    assert ts(2, 8, 16, F32, P, NULL, P, 5, P, None) == EINVAL
    assert ts(-2, 8, 16, F32, P, NULL, P, 3, P, None) == EINVAL
    assert ts(2, 8, 16, 4, P, NULL, P, 3, P, None) == EDTYPE
    assert ts(2, 8, 16, F32, NULL, NULL, P, 3, P, None) == EINVAL
    assert ts(2, 8, 16, F32, P, NULL, NULL, 3, P, None) == EINVAL
    assert ts(2, 8, 16, F32, P, NULL, P, 3, NULL, None) == EINVAL
    assert ts(2, 0, 16, F32, NULL, NULL, NULL, 3, NULL, None) == OK
    fg = lib.wkv_forward_gated
    assert fg(2, 300, 64, F32, P, P, P, P, NULL, P, NULL, 0, P, 1 << 30, None) == EINVAL
    need = lib.wkv_saved_states_bytes(2, 300, 64)
    assert fg(2, 300, 64, F32, P, P, P, P, P, P, P, need - 1, P, 1 << 30, None) == EINVAL
    assert fg(2, 300, 64, 3, P, P, P, P, P, P, NULL, 0, P, 1 << 30, None) == EDTYPE
    assert fg(0, 300, 64, F32, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, None) == OK
    bg = lib.wkv_backward_gated
    wsb = lib.wkv_backward_workspace_bytes(2, 300, 64, F32)
    ptrs = [P] * 4 + [NULL] + [P] + [NULL, 0] + [P] * 5
    assert bg(2, 300, 64, F32, *ptrs, P, wsb, None) == EINVAL  # r missing
    ptrs = [P] * 6 + [NULL, 0] + [P, P, NULL, P, P]
    assert bg(2, 300, 64, F32, *ptrs, P, wsb, None) == EINVAL  # gr missing
    ptrs = [P] * 6 + [NULL, 0] + [P] * 5
    assert bg(2, 300, 64, F32, *ptrs, P, wsb - 1, None) == EWS


def test_token_shift_backward_argument_checks():
    def tsb(B, T, C, dt=F32, M=3, x=P, xp=NULL, mu=P, g=P, gx=P, gmu=P, gp=P, ws=P, wsb=1 << 30):
        return lib.wkv_token_shift_backward(B, T, C, dt, x, xp, mu, M, g, gx, gmu, gp, ws, wsb, None)
    assert tsb(-1, 4, 4) == EINVAL
    assert tsb(1, 4, 4, M=0) == EINVAL
    assert tsb(1, 4, 4, M=5) == EINVAL
    assert tsb(1, 4, 4, dt=9) == EDTYPE
    for kw in ({"x": NULL}, {"g": NULL}, {"gx": NULL}, {"mu": NULL}, {"gmu": NULL}):
        assert tsb(1, 4, 4, **kw) == EINVAL, kw
    need = lib.wkv_token_shift_backward_workspace_bytes(2, 100, 64, 3)
    assert need >= 4 * 3 * 2 * 64 * 4  # four 32-step segments of partial sums per (mix, lane)
    assert tsb(2, 100, 64, ws=NULL, wsb=0) == EWS
    assert tsb(2, 100, 64, wsb=need - 1) == EWS
    assert lib.wkv_token_shift_backward_workspace_bytes(2, 100, 64, 0) == ctypes.c_size_t(-1).value
    assert lib.wkv_token_shift_backward_workspace_bytes(2, 0, 64, 3) == 0
    assert tsb(0, 4, 4, x=NULL, g=NULL, gx=NULL, ws=NULL, wsb=0) == OK  # empty: nothing to do


def test_linear_attention_argument_checks():
    la = lib.wkv_linear_attention
    q = lib.wkv_linear_attention_workspace_bytes
    bad = ctypes.c_size_t(-1).value
    assert q(4, 100, 32, 32, F32) > 0 and q(4, 100, 48, 48, F32) == bad and q(4, 100, 16, 16, F32) == bad
    for D, M in ((32, 64), (64, 32), (64, 64)):  # D and M each 32 or 64
        assert q(4, 100, D, M, F32) > 0 and q(4, 100, D, M, BF16) > 0
    assert q(4, 100, 32, 48, F32) == bad and q(4, 100, 128, 64, F32) == bad
    assert q(-1, 100, 32, 32, F32) == bad and q(4, 100, 32, 32, 7) == bad and q(0, 100, 32, 32, F32) == 0
    need = q(4, 100, 32, 32, BF16)
    assert la(4, 100, 48, 48, F32, P, P, P, P, 1, P, need, None) == EINVAL
    assert la(4, 100, 32, 32, 9, P, P, P, P, 1, P, need, None) == EDTYPE
    lx = lib.wkv_linear_attention_ex
    assert lx(4, 100, 32, 32, F32, P, P, P, P, 1, P, need, 3, None) == EINVAL  # unknown algorithm
    assert lx(4, 100, 32, 32, F32, P, P, P, P, 1, P, need - 1, 2, None) == EWS
    assert lx(0, 100, 32, 32, F32, NULL, NULL, NULL, NULL, 1, NULL, 0, 1, None) == OK
    # one workspace serves both evaluations: records for the one pass and the aggregates for the
    # three launches (per chunk of 512 positions, both dtypes: 2 x 1056 tagged words and 1056
    # floats)
    chunks = 64 * 32
    assert q(64, 16384, 32, 32, F32) >= chunks * 1056 * (2 * 8 + 4)
    assert q(64, 16384, 32, 32, BF16) >= chunks * 1056 * (2 * 8 + 4)
    assert la(-4, 100, 32, 32, F32, P, P, P, P, 1, P, need, None) == EINVAL
    assert la(4, 100, 32, 32, F32, NULL, P, P, P, 1, P, need, None) == EINVAL
    assert la(4, 100, 32, 32, F32, P, P, P, NULL, 1, P, need, None) == EINVAL
    assert la(4, 100, 32, 32, F32, P, P, P, P, 1, NULL, 0, None) == EWS
    assert la(4, 100, 32, 32, F32, P, P, P, P, 1, P, need - 1, None) == EWS
    assert la(0, 100, 32, 32, F32, NULL, NULL, NULL, NULL, 1, NULL, 0, None) == OK
    # q, k, v, out must be 16-byte aligned; checked before anything is launched
    odd = ctypes.c_void_p(P.value + 8)
    for i in range(4):
        args = [P, P, P, P]
        args[i] = odd
        assert la(4, 100, 32, 32, BF16, *args, 1, P, need, None) == EINVAL
        assert lx(4, 100, 32, 32, F32, *args, 1, P, need, 2, None) == EINVAL


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib

    monkeypatch.setattr(libwkv, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        libwkv._load()
    importlib.reload(libwkv)  # restore the real module state


def test_binding_refuses_host_tensors():
    """Every wrapper refuses host tensors before any GPU call (the C ABI takes raw device pointers
    and cannot tell them apart); the same checks with one host tensor among GPU ones run in
    tests/test_binding_gpu.py."""
    import torch

    B, T, C, M = 2, 8, 4, 3
    w, u, k, v, gy, r = (torch.ones(C), torch.zeros(C), torch.zeros(B, T, C), torch.zeros(B, T, C),
                         torch.zeros(B, T, C), torch.zeros(B, T, C))
    a, b, p = torch.zeros(B, 1, C), torch.zeros(B, 1, C), torch.zeros(B, 1, C)
    mu, gm = torch.rand(M, C), torch.zeros(M, B, T, C)
    ws = torch.zeros(1 << 12, dtype=torch.uint8)
    calls = [
        lambda: libwkv.wkv_forward(w, u, k, v),
        lambda: libwkv.wkv_forward_noalloc(w, u, k, v),
        lambda: libwkv.wkv_step(w.view(1, C), u.view(1, C), k[:, :1].contiguous(), v[:, :1].contiguous(), a, b, p),
        lambda: libwkv.wkv_forward_save(w, u, k, v),
        lambda: libwkv.wkv_backward(w, u, k, v, gy),
        lambda: libwkv.wkv_forward_gated(w, u, k, v, r),
        lambda: libwkv.wkv_backward_gated(w, u, k, v, r, gy),
        lambda: libwkv.wkv_token_shift(k, mu),
        lambda: libwkv.wkv_token_shift_backward(k, mu, gm),
        lambda: libwkv.linear_attention(torch.zeros(2, 8, 32), torch.zeros(2, 8, 32), torch.zeros(2, 8, 32)),
        lambda: libwkv.wkv_forward_workspace_init(ws),
        lambda: libwkv.workspace_query(ws),
        lambda: libwkv.force_give_up(ws),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError):
            call()
