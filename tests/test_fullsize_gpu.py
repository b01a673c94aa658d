"""The full-size workloads, in the launch configuration the benchmark times.

Forward workloads compare every output with the float64 recurrence and sampled
(lane, t) outputs with the direct sums.  The decode workload (256 x 32 x 4096
lanes, 128 prefix steps then 16 timed steps) compares 4096 sampled lanes over
all 144 steps with the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import scaled_error, state_log_b, wkv_direct_at, wkv_recurrent
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TOL, host, run_forward, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def forward_fullsize(spec, algos):
    print(f"  {spec.name}: generating", flush=True)
    inp = workloads.forward_inputs(spec)
    dev = to_device(inp)
    ys = {}
    for algo in algos:
        ys[algo] = host(run_forward(dev, algo)).astype(np.float32)
        print(f"  {spec.name}: {algo} done", flush=True)
    del dev
    torch.cuda.empty_cache()
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    print(f"  {spec.name}: oracle done", flush=True)
    for algo, y in ys.items():
        err = scaled_error(y, y_ref, s_ref)
        print(f"  {spec.name} {algo}: scaled error {err:.3e}", flush=True)
        assert err <= TOL[spec.dtype], (algo, err)
        for (b, c) in workloads.sample_lanes(spec.B, spec.C, 6, seed=7):
            for t in (0, spec.T // 3, spec.T - 1):
                yt, st = wkv_direct_at(inp["w"][c], inp["u"][c], inp["k"][b, :, c], inp["v"][b, :, c], t)
                assert abs(float(y[b, t, c]) - yt) <= TOL[spec.dtype] * st, (algo, b, c, t)


def test_ctx8192_width2048_f32():
    forward_fullsize(workloads.FWD_CTX8K, ["auto", "seq"])


def test_ctx65536_width5120_bf16():
    forward_fullsize(workloads.FWD_LONG_BF16, ["auto"])


def test_decode_256x32x4096():
    spec = workloads.STEP_DECODE
    N, G, C = spec.N, spec.G, spec.C
    w, u = workloads.step_params(spec)
    wd, ud = torch.from_numpy(w).cuda(), torch.from_numpy(u).cuda()
    a, b, p = libwkv.empty_state((N, G, C))
    lanes = torch.from_numpy(np.random.default_rng(3).choice(N * G * C, 4096, replace=False)).cuda()
    total = spec.prefix + spec.steps
    ks, vs, ys = [], [], []
    for s in range(total):
        k, v = workloads.step_kv(spec, s, device="cuda")
        y = libwkv.wkv_step(wd, ud, k, v, a, b, p)
        ks.append(host(k.view(-1)[lanes]))
        vs.append(host(v.view(-1)[lanes]))
        ys.append(host(y.view(-1)[lanes]))
    torch.cuda.synchronize()
    li = lanes.cpu().numpy()
    wl, ul = w.reshape(-1)[li % (G * C)], u.reshape(-1)[li % (G * C)]
    kk = np.stack(ks)[None]  # [1, steps, lanes]
    vv = np.stack(vs)[None]
    y_ref, s_ref, (ra, rb, rp) = wkv_recurrent(wl, ul, kk, vv, return_scale=True, return_state=True)
    y = np.stack(ys)[None]
    err = scaled_error(y[:, spec.prefix:], y_ref[:, spec.prefix:], s_ref[:, spec.prefix:])
    print(f"  decode: scaled error over the timed steps {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert scaled_error(y, y_ref, s_ref) <= TOL["bf16"]
    ga, gb, gp = (host(x.view(-1)[lanes]) for x in (a, b, p))
    np.testing.assert_allclose(state_log_b(ga, gb, gp), state_log_b(ra, rb, rp)[0], rtol=0, atol=2e-5)
