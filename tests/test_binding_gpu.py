"""The binding refuses tensors that would hand a kernel a host or misshapen buffer.

Every wrapper passes raw device pointers through the C ABI, which cannot tell a host pointer from
a device one, so each tensor argument (inputs, caller-given outputs, workspaces, saved states)
must be a contiguous tensor on the current GPU, and caller-given outputs must have the shape and
dtype the call writes.  Here one argument at a time is a host tensor or has the wrong shape while
the rest are valid GPU tensors; the library's launching entry points are replaced by a stub for
the duration, so a refusal that came too late fails the test without reaching the GPU.  The
last test makes the same calls with valid arguments through the real library.
"""
import pytest
import torch

from rwkv_linear_attention_libwkv_amd import libwkv

pytestmark = pytest.mark.gpu

B, T, C = 2, 80, 64

# host-side queries, and the workspace fill the wrappers issue for the workspaces they allocate
PASS_THROUGH = ("_bytes", "wkv_status_string", "wkv_forward_workspace_init")


class LaunchStub:
    def __init__(self, real):
        self.real = real
        self.launched = []

    def __getattr__(self, name):
        fn = getattr(self.real, name)
        if name.endswith(PASS_THROUGH):
            return fn

        def stub(*args):
            self.launched.append(name)
            raise AssertionError(f"{name} was called with arguments the binding should have refused")

        return stub


@pytest.fixture
def stub(monkeypatch):
    s = LaunchStub(libwkv.lib)
    monkeypatch.setattr(libwkv, "lib", s)
    return s


def g(*shape, dtype=torch.float32):
    return torch.randn(shape, device="cuda").to(dtype)


def h(*shape, dtype=torch.float32):
    return torch.randn(shape).to(dtype)


def refused(fn, stub):
    with pytest.raises(ValueError):
        fn()
    assert stub.launched == []


def test_forward_family(stub):
    w, u, k, v = g(C).exp(), g(C), g(B, T, C), g(B, T, C)
    refused(lambda: libwkv.wkv_forward(w, u, k, v, y=h(B, T, C)), stub)
    refused(lambda: libwkv.wkv_forward(w, u, k, v, algo="chunked", workspace=h(1 << 20, dtype=torch.uint8)), stub)
    refused(lambda: libwkv.wkv_forward(w, u, k, v, state=(h(B, C), g(B, C), g(B, C))), stub)
    refused(lambda: libwkv.wkv_forward(w, u, k, v, return_state=True, state_out=(g(B, C), h(B, C), g(B, C))), stub)
    refused(lambda: libwkv.wkv_forward_noalloc(w, u, k, v, y=h(B, T, C)), stub)
    refused(lambda: libwkv.wkv_forward_noalloc(h(C), u, k, v), stub)
    refused(lambda: libwkv.wkv_forward_save(w, u, k, v, saved=h(1 << 20, dtype=torch.uint8)), stub)
    refused(lambda: libwkv.wkv_forward_save(w, h(C), k, v), stub)
    refused(lambda: libwkv.wkv_forward_gated(w, u, k, v, h(B, T, C)), stub)
    refused(lambda: libwkv.wkv_forward_gated(w, u, k, v, g(B, T, C), z=h(B, T, C)), stub)


def test_step(stub):
    N, G = 4, 2
    w, u = g(G, C).exp(), g(G, C)
    k, v = g(N, G, C), g(N, G, C)
    a, b, p = libwkv.empty_state((N, G, C))
    refused(lambda: libwkv.wkv_step(w, u, h(N, G, C), v, a, b, p), stub)
    refused(lambda: libwkv.wkv_step(h(G, C), u, k, v, a, b, p), stub)
    refused(lambda: libwkv.wkv_step(w, u, k, v, a, b, p, y=h(N, G, C)), stub)


def test_backward_family(stub):
    w, u, k, v, gy = g(C).exp(), g(C), g(B, T, C), g(B, T, C), g(B, T, C)
    refused(lambda: libwkv.wkv_backward(w, u, k, v, gy, gk=h(B, T, C)), stub)
    refused(lambda: libwkv.wkv_backward(w, u, k, v, gy, gw=h(B, C)), stub)
    refused(lambda: libwkv.wkv_backward(w, u, k, v, gy, saved=h(1 << 20, dtype=torch.uint8)), stub)
    refused(lambda: libwkv.wkv_backward(w, u, k, v, gy, workspace=h(1 << 20, dtype=torch.uint8)), stub)
    r = g(B, T, C)
    refused(lambda: libwkv.wkv_backward_gated(w, u, k, v, r, gy, gr=h(B, T, C)), stub)
    refused(lambda: libwkv.wkv_backward_gated(w, u, k, v, r, gy, gr=g(B, T, C + 1)), stub)
    refused(lambda: libwkv.wkv_backward_gated(w, u, k, v, r, gy, gw=g(B, C - 1)), stub)
    refused(lambda: libwkv.wkv_backward_gated(h(C), u, k, v, r, gy), stub)
    refused(lambda: libwkv.wkv_backward_gated(g(C + 1), u, k, v, r, gy), stub)


def test_token_shift_family(stub):
    M = 3
    x, mu, gg = g(B, T, C), torch.rand(M, C, device="cuda"), g(M, B, T, C)
    refused(lambda: libwkv.wkv_token_shift(x, h(M, C)), stub)
    refused(lambda: libwkv.wkv_token_shift(x, mu, x_prev=h(B, C)), stub)
    refused(lambda: libwkv.wkv_token_shift(x, mu, out=h(M, B, T, C)), stub)
    refused(lambda: libwkv.wkv_token_shift_backward(x, mu, gg, gx=h(B, T, C)), stub)
    refused(lambda: libwkv.wkv_token_shift_backward(x, mu, gg, gmu=g(M, B, C + 1)), stub)
    refused(lambda: libwkv.wkv_token_shift_backward(x, mu, gg, gprev=g(B + 1, C)), stub)
    refused(lambda: libwkv.wkv_token_shift_backward(x, mu, gg, workspace=h(1 << 20, dtype=torch.uint8)), stub)


def test_linear_attention_and_workspace_tools(stub):
    q, k, v = g(2, 100, 32), g(2, 100, 32), g(2, 100, 32)
    refused(lambda: libwkv.linear_attention(q, k, v, out=h(2, 100, 32)), stub)
    refused(lambda: libwkv.linear_attention(q, k, v, workspace=h(1 << 20, dtype=torch.uint8)), stub)
    host_ws = h(1 << 16, dtype=torch.uint8)
    refused(lambda: libwkv.workspace_query(host_ws), stub)
    refused(lambda: libwkv.force_give_up(host_ws), stub)
    refused(lambda: libwkv.wkv_forward_workspace_init(host_ws), stub)


def test_valid_calls_after_refusals():
    """The same wrappers with valid arguments run (the refusals above left nothing behind)."""
    w, u, k, v, gy = g(C).exp(), g(C), g(B, T, C), g(B, T, C), g(B, T, C)
    y = libwkv.wkv_forward(w, u, k, v, algo="chunked")
    y_ref = libwkv.wkv_forward(w, u, k, v, algo="seq")
    torch.cuda.synchronize()
    assert torch.allclose(y, y_ref, rtol=1e-5, atol=1e-5)
    gw, gu, gk, gv = libwkv.wkv_backward(w, u, k, v, gy)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all() for t in (gw, gu, gk, gv))
