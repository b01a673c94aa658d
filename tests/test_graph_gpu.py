"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The chunked scans keep launch counters in their workspace, set by kernels (never a memset), and
every launch's last workgroup resets them for the next; a replayed graph must therefore behave
like the same launches made eagerly.  Each case computes eager results for two input sets, then
captures the call on static buffers and replays it several times, loading one input set or the
other into the static buffers before each replay, with the program's own eager work and a
synchronisation between replays; every replay must give bitwise the eager result of its input
set (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

from rwkv_linear_attention_libwkv_amd import libwkv, workloads

pytestmark = pytest.mark.gpu

REPLAYS = 6


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dtype)


def capture(fn):
    """fn() captured in a graph, after two warm-up calls on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def eager_noise():
    """Unrelated eager work between replays: a forward of its own and some torch ops."""
    spec = workloads.FWD_SMALL.with_(B=1, T=700, C=64, seed=99)
    inp = workloads.forward_inputs(spec)
    y = libwkv.wkv_forward(dev(inp["w"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), algo="chunked")
    (y * 2.0 + 1.0).relu_()
    torch.cuda.synchronize()


def replay_and_check(graph, load, outputs, expected):
    """Replay with input set i % 2 loaded; outputs() must equal expected[i % 2] bit for bit."""
    for i in range(REPLAYS):
        load(i % 2)
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for a, b in zip(got, expected[i % 2]):
            assert torch.equal(a, b), f"replay {i}"
        eager_noise()


def forward_sets(B, T, C, dtype, seeds):
    sets = []
    for s in seeds:
        inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, dtype=dtype, seed=s))
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        sets.append({n: dev(inp[n], tdt if n in ("k", "v") else torch.float32) for n in ("w", "u", "k", "v")})
    return sets


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_chunked(dtype):
    B, T, C = 2, 1500, 96
    sets = forward_sets(B, T, C, dtype, (31, 32))
    expected = [[libwkv.wkv_forward(s["w"], s["u"], s["k"], s["v"], algo="chunked").clone()] for s in sets]
    st = {n: sets[0][n].clone() for n in sets[0]}
    y = torch.empty_like(st["k"])
    ws = libwkv.new_workspace(B, T, C, st["k"].dtype, "chunked")
    torch.cuda.synchronize()
    graph = capture(lambda: libwkv.wkv_forward(st["w"], st["u"], st["k"], st["v"], algo="chunked", y=y,
                                               workspace=ws))

    def load(i):
        for n in st:
            st[n].copy_(sets[i][n])

    replay_and_check(graph, load, lambda: [y], expected)
    assert libwkv.lookback_error(ws) == 0


def test_forward_noalloc():
    B, T, C = 2, 2000, 64
    sets = forward_sets(B, T, C, "bf16", (33, 34))
    expected = [[libwkv.wkv_forward(s["w"], s["u"], s["k"], s["v"]).clone()] for s in sets]
    st = {n: sets[0][n].clone() for n in sets[0]}
    y = torch.empty_like(st["k"])
    libwkv.wkv_forward_noalloc(st["w"], st["u"], st["k"], st["v"], y=y)  # first call on the device: set-up
    torch.cuda.synchronize()
    graph = capture(lambda: libwkv.wkv_forward_noalloc(st["w"], st["u"], st["k"], st["v"], y=y))

    def load(i):
        for n in st:
            st[n].copy_(sets[i][n])

    replay_and_check(graph, load, lambda: [y], expected)


def test_decode_steps():
    """Eight decode steps in one graph, from a state restored before every replay."""
    N, G, C, S = 16, 4, 256, 8
    rng = np.random.default_rng(35)
    w = dev(np.exp(rng.uniform(-3, 1, (G, C))))
    u = dev(rng.normal(0, 0.5, (G, C)))
    kv = [[(dev(rng.normal(0, 1, (N, G, C)), torch.bfloat16), dev(rng.normal(0, 1, (N, G, C)), torch.bfloat16))
           for _ in range(S)] for _ in range(2)]
    start = [tuple(dev(x) for x in (rng.normal(0, 1, (N, G, C)), rng.uniform(0.5, 2, (N, G, C)),
                                    rng.normal(0, 1, (N, G, C)))) for _ in range(2)]
    expected = []
    for i in range(2):
        a, b, p = (x.clone() for x in start[i])
        ys = [libwkv.wkv_step(w, u, k, v, a, b, p).clone() for k, v in kv[i]]
        expected.append(ys + [a, b, p])
    sk = [(k.clone(), v.clone()) for k, v in kv[0]]
    a, b, p = (x.clone() for x in start[0])
    ys = [torch.empty_like(sk[0][0]) for _ in range(S)]
    torch.cuda.synchronize()

    def decode():
        for (k, v), y in zip(sk, ys):
            libwkv.wkv_step(w, u, k, v, a, b, p, y=y)

    graph = capture(decode)

    def load(i):
        for (k, v), (k0, v0) in zip(sk, kv[i]):
            k.copy_(k0)
            v.copy_(v0)
        for x, x0 in zip((a, b, p), start[i]):
            x.copy_(x0)

    replay_and_check(graph, load, lambda: ys + [a, b, p], expected)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_training_pair(dtype):
    """wkv_forward_save then wkv_backward_saved in one graph."""
    B, T, C = 2, 900, 64
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    sets = forward_sets(B, T, C, dtype, (36, 37))
    for i, s in enumerate(sets):
        s["gy"] = dev(np.random.default_rng(38 + i).normal(0, 1, (B, T, C)), tdt)
    expected = []
    for s in sets:
        y, saved = libwkv.wkv_forward_save(s["w"], s["u"], s["k"], s["v"])
        expected.append([y.clone()] + [g.clone() for g in libwkv.wkv_backward(s["w"], s["u"], s["k"], s["v"], s["gy"],
                                                                                saved=saved)])
    st = {n: sets[0][n].clone() for n in sets[0]}
    y = torch.empty_like(st["k"])
    saved = torch.empty(libwkv.wkv_saved_states_bytes(B, T, C), dtype=torch.uint8, device="cuda")
    fws = libwkv.new_workspace(B, T, C, tdt, "chunked")
    bws = libwkv.new_backward_workspace(B, T, C, tdt)
    gk, gv = torch.empty_like(y), torch.empty_like(y)
    gw, gu = (torch.empty((B, C), device="cuda") for _ in range(2))
    torch.cuda.synchronize()

    def pair():
        libwkv.wkv_forward_save(st["w"], st["u"], st["k"], st["v"], y=y, saved=saved, workspace=fws)
        libwkv.wkv_backward(st["w"], st["u"], st["k"], st["v"], st["gy"], saved=saved, gk=gk, gv=gv, gw=gw, gu=gu,
                            workspace=bws)

    graph = capture(pair)

    def load(i):
        for n in st:
            st[n].copy_(sets[i][n])

    replay_and_check(graph, load, lambda: [y, gw, gu, gk, gv], expected)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linear_attention_one_pass(dtype):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    sets = []
    for s in (40, 41):
        inp = workloads.linear_attention_inputs(workloads.LA_SMALL.with_(BH=4, N=1300, dtype=dtype, seed=s))
        sets.append({n: dev(inp[n], tdt) for n in ("q", "k", "v")})
    expected = [[libwkv.linear_attention(s["q"], s["k"], s["v"], algo="one").clone()] for s in sets]
    st = {n: sets[0][n].clone() for n in sets[0]}
    out = torch.empty_like(st["v"])
    ws = libwkv.new_la_workspace(4, 1300, 32, 32, tdt)
    torch.cuda.synchronize()
    graph = capture(lambda: libwkv.linear_attention(st["q"], st["k"], st["v"], out=out, workspace=ws, algo="one"))

    def load(i):
        for n in st:
            st[n].copy_(sets[i][n])

    replay_and_check(graph, load, lambda: [out], expected)


def test_token_shift_and_backward():
    B, T, C, M = 2, 600, 96, 3
    rng = np.random.default_rng(42)
    sets = [{"x": dev(rng.normal(0, 1, (B, T, C))), "g": dev(rng.normal(0, 1, (M, B, T, C)))} for _ in range(2)]
    mu = dev(rng.uniform(0, 1, (M, C)))
    expected = []
    for s in sets:
        out = libwkv.wkv_token_shift(s["x"], mu).clone()
        expected.append([out] + [t.clone() for t in libwkv.wkv_token_shift_backward(s["x"], mu, s["g"])])
    st = {n: sets[0][n].clone() for n in sets[0]}
    out = torch.empty((M, B, T, C), device="cuda")
    gx, gmu, gprev = torch.empty((B, T, C), device="cuda"), torch.empty((M, B, C), device="cuda"), torch.empty(
        (B, C), device="cuda")
    sws = torch.empty(libwkv.lib.wkv_token_shift_backward_workspace_bytes(B, T, C, M), dtype=torch.uint8,
                      device="cuda")
    torch.cuda.synchronize()

    def both():
        libwkv.wkv_token_shift(st["x"], mu, out=out)
        libwkv.wkv_token_shift_backward(st["x"], mu, st["g"], gx=gx, gmu=gmu, gprev=gprev, workspace=sws)

    graph = capture(both)

    def load(i):
        for n in st:
            st[n].copy_(sets[i][n])

    replay_and_check(graph, load, lambda: [out, gx, gmu, gprev], expected)


FIRST_CALL_CAPTURED = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from rwkv_linear_attention_libwkv_amd import libwkv, workloads

# the process's first call into the library is made under capture: the per-device lookups the
# chunked forward makes on its first launch (compute units, resident workgroups) happen inside it
inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=2, T=1500, C=128, seed=4))
t = lambda a: torch.from_numpy(a).cuda()
w, u, k, v = t(inp["w"]), t(inp["u"]), t(inp["k"]), t(inp["v"])
y = torch.empty_like(k)
ws = libwkv.new_workspace(2, 1500, 128, torch.float32, "chunked", 256)
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    lib = libwkv.lib
    st = lib.wkv_forward_ex(2, 1500, 128, 0, w.data_ptr(), u.data_ptr(), k.data_ptr(), v.data_ptr(),
                            y.data_ptr(), ws.data_ptr(), ws.numel(), 2, 256, torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
torch.cuda.synchronize()
outs = []
for _ in range(3):
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    outs.append(y.clone())
ref = libwkv.wkv_forward(w, u, k, v, algo="chunked", chunk_len=256)
torch.cuda.synchronize()
assert all(torch.equal(o, ref) for o in outs)
print("first call captured: ok", flush=True)
"""


def test_first_call_under_capture(tmp_path):
    """In a fresh process whose first call into the library is captured, the capture succeeds and
    every replay equals the eager call bit for bit (a child process, so that nothing earlier in
    this one has made the first launch)."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "first_call.py"
    script.write_text(FIRST_CALL_CAPTURED)
    r = subprocess.run([sys.executable, str(script), root], capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "first call captured: ok" in r.stdout
