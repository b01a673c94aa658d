"""GPU parity of wkv_step (RNN-mode decoding) against the float64 oracle.

A run of steps over lanes (n, g, c) is the forward recurrence of B = N
sequences over G*C channels, so the oracle's wkv_recurrent supplies y and the
scale s for every step; wkv_step_ref checks single steps from arbitrary states.
"""
import numpy as np
import pytest
import torch

from oracle import EMPTY_P, scaled_error, state_log_b, state_ratio, wkv_recurrent, wkv_step_ref
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TOL, TORCH_DT, host, run_forward

pytestmark = pytest.mark.gpu


def decode_run(spec, dtype):
    """Run spec.prefix + spec.steps steps from the empty state on the GPU; oracle alongside."""
    w, u = workloads.step_params(spec)
    N, G, C = spec.N, spec.G, spec.C
    wd, ud = torch.from_numpy(w).cuda(), torch.from_numpy(u).cuda()
    a, b, p = libwkv.empty_state((N, G, C))
    total = spec.prefix + spec.steps
    ks, vs, ys = [], [], []
    for s in range(total):
        k, v = workloads.step_kv(spec, s, device="cuda")
        k, v = k.to(TORCH_DT[dtype]), v.to(TORCH_DT[dtype])
        ys.append(host(libwkv.wkv_step(wd, ud, k, v, a, b, p)))
        ks.append(host(k))
        vs.append(host(v))
    torch.cuda.synchronize()
    kk = np.stack(ks, axis=1).reshape(N, total, G * C)
    vv = np.stack(vs, axis=1).reshape(N, total, G * C)
    y_ref, s_ref, (ra, rb, rp) = wkv_recurrent(w.reshape(-1), u.reshape(-1), kk, vv,
                                               return_scale=True, return_state=True)
    y = np.stack(ys, axis=1).reshape(N, total, G * C)
    return y, y_ref, s_ref, (host(a), host(b), host(p)), (ra, rb, rp)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_match_recurrence(dtype):
    spec = workloads.STEP_DECODE.with_(N=8, G=4, C=256, prefix=24, steps=8)
    y, y_ref, s_ref, (a, b, p), (ra, rb, rp) = decode_run(spec, dtype)
    err = scaled_error(y, y_ref, s_ref)
    print(f"  step {dtype}: scaled error {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    # the stored state is the oracle's state (compared through its invariants)
    a, b, p = (x.reshape(spec.N, -1) for x in (a, b, p))
    np.testing.assert_allclose(state_log_b(a, b, p), state_log_b(ra, rb, rp), rtol=0, atol=2e-5)
    np.testing.assert_allclose(state_ratio(a, b, p), state_ratio(ra, rb, rp), rtol=0, atol=2e-5 * 5)


def test_single_step_from_arbitrary_states():
    rng = np.random.default_rng(5)
    N, G, C = 4, 3, 128
    w = np.exp(rng.uniform(-3, 1, (G, C))).astype(np.float32)
    u = rng.normal(0, 0.5, (G, C)).astype(np.float32)
    k = rng.normal(0, 2, (N, G, C)).astype(np.float32)
    v = rng.normal(0, 1, (N, G, C)).astype(np.float32)
    a = rng.normal(0, 1, (N, G, C)).astype(np.float32)
    b = rng.uniform(0.3, 3, (N, G, C)).astype(np.float32)
    p = rng.normal(0, 5, (N, G, C)).astype(np.float32)
    p[0, 0, :7], a[0, 0, :7], b[0, 0, :7] = EMPTY_P, 0, 0  # empty lanes: y = v
    k[1, 1, :5] += 150.0  # exponent far above the state's
    p[2, 2, :5] += 150.0  # state far above the token's
    y_ref, (ra, rb, rp) = wkv_step_ref(w, u, k, v, a, b, p)
    t = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
    ga, gb, gp = t(a), t(b), t(p)
    y = host(libwkv.wkv_step(t(w), t(u), t(k), t(v), ga, gb, gp))
    # scale: the same weights applied to |a| / b and |v|
    uk = u + k
    q = np.maximum(p, uk)
    e1, e2 = np.exp(p.astype(np.float64) - q), np.exp(uk.astype(np.float64) - q)
    s = (e1 * np.abs(a) + e2 * np.abs(v)) / (e1 * b + e2)
    assert scaled_error(y, y_ref, s) <= 2e-5
    np.testing.assert_array_equal(y[0, 0, :7], v[0, 0, :7])
    ga, gb, gp = host(ga), host(gb), host(gp)
    np.testing.assert_allclose(state_log_b(ga, gb, gp), state_log_b(ra, rb, rp), rtol=0, atol=2e-5)
    np.testing.assert_allclose(state_ratio(ga, gb, gp), state_ratio(ra, rb, rp), rtol=0,
                               atol=2e-5 * np.abs(state_ratio(ra, rb, rp)).max())


def test_prefill_then_decode():
    """wkv_forward with state out, then wkv_step, equals one long forward (the modes hand over)."""
    spec = workloads.FWD_SMALL.with_(B=3, T=400, C=128, k_std=2.0, seed=21)
    inp = workloads.forward_inputs(spec)
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    w, u = torch.from_numpy(inp["w"]).cuda(), torch.from_numpy(inp["u"]).cuda()
    k, v = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    T1 = 300
    dev = {"w": w, "u": u, "k": k[:, :T1].contiguous(), "v": v[:, :T1].contiguous()}
    y1, (a, b, p) = run_forward(dev, "chunked", 128, return_state=True)
    ys = [host(y1)]
    a, b, p = (x.reshape(3, 1, 128).contiguous() for x in (a, b, p))
    for t in range(T1, spec.T):
        kt = k[:, t].reshape(3, 1, 128).contiguous()
        vt = v[:, t].reshape(3, 1, 128).contiguous()
        ys.append(host(libwkv.wkv_step(w.view(1, 128), u.view(1, 128), kt, vt, a, b, p)).reshape(3, 1, 128))
    y = np.concatenate(ys, axis=1)
    assert scaled_error(y, y_ref, s_ref) <= TOL["f32"]
