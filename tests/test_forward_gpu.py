"""GPU parity of wkv_forward (both algorithms) against the float64 oracle.

Gate: scale-normalised error max |y_gpu - y| / s (s = the convex weights applied
to |v|) at most 2e-5 for float32 and 1e-2 for bfloat16 k, v, y.
"""
import numpy as np
import pytest
import torch

from oracle import scaled_error, wkv_direct, wkv_direct_at, wkv_recurrent
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from rwkv_linear_attention_libwkv_amd.workloads import round_to_bf16
from tests.gpu_util import TOL, host, run_forward, to_device

pytestmark = pytest.mark.gpu

ALGOS = [("seq", 0), ("chunked", 64), ("chunked", 128), ("chunked", 256)]


def check(inp, algos=ALGOS, direct=False):
    if direct:
        y_ref, s_ref = wkv_direct(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    else:
        y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    dev = to_device(inp)
    for algo, cl in algos:
        y = host(run_forward(dev, algo, cl))
        err = scaled_error(y, y_ref, s_ref)
        print(f"  {algo:8s} chunk {cl:3d}: scaled error {err:.3e}", flush=True)
        assert err <= TOL[inp["dtype"]], (algo, cl, err)


def test_small_workload_all_algorithms():
    """B=1, T=64, C=64 float32 against the direct O(T^2) sums."""
    check(workloads.forward_inputs(workloads.FWD_SMALL), direct=True)


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 1, 7), (1, 2, 3), (3, 127, 100), (2, 129, 65),
                                   (1, 257, 130), (2, 300, 64), (1, 700, 1)])
def test_ragged_shapes(B, T, C):
    check(workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, seed=B * 1000 + T + C)))


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_tile_boundaries(chunk):
    for T in (chunk - 1, chunk, chunk + 1, 3 * chunk + 5):
        inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=2, T=T, C=70, seed=T))
        check(inp, algos=[("chunked", chunk), ("seq", 0)])


def test_169m_width_workload():
    """B=8, T=1024, C=768 float32: full tensor against the recurrence, samples against the sums."""
    spec = workloads.FWD_169M
    inp = workloads.forward_inputs(spec)
    check(inp, algos=[("auto", 0), ("seq", 0), ("chunked", 128), ("chunked", 256)])
    dev = to_device(inp)
    y = host(run_forward(dev))
    for (b, c) in workloads.sample_lanes(spec.B, spec.C, 8):
        for t in (0, 1, 511, spec.T - 1):
            yt, st = wkv_direct_at(inp["w"][c], inp["u"][c], inp["k"][b, :, c], inp["v"][b, :, c], t)
            assert abs(y[b, t, c] - yt) <= TOL["f32"] * st


def test_bf16_io():
    """bfloat16 k, v, y with float32 state on a shortened long-context workload (chunk 0 is the
    default tile, 512 tokens for bfloat16 row pairs)."""
    inp = workloads.forward_inputs(workloads.FWD_LONG_BF16.with_(T=2048, C=512))
    check(inp, algos=[("seq", 0), ("chunked", 0), ("chunked", 128), ("chunked", 256), ("chunked", 512)])


@pytest.mark.parametrize("k_std", [2.5, 4.0, 6.0])
def test_bf16_pairs_wide_key_ranges(k_std):
    """bfloat16 row pairs with wide key spreads: waves whose keys span more than the fast path's
    range walk their tokens exactly, so these spreads mix both kinds of wave within tiles and
    along the chain."""
    inp = workloads.forward_inputs(workloads.FWD_LONG_BF16.with_(B=2, T=3000, C=128, k_std=k_std, seed=31))
    check(inp, algos=[("chunked", 0), ("chunked", 256)])


def test_bf16_pairs_all_negative_keys():
    """Every key negative (the chunk reference is then the key of smallest magnitude)."""
    inp = workloads.forward_inputs(workloads.FWD_LONG_BF16.with_(B=1, T=2100, C=128, seed=32))
    inp["k"] = workloads.round_to_bf16(-np.abs(inp["k"]) - np.float32(0.25))
    check(inp, algos=[("chunked", 0), ("seq", 0)])


def test_bf16_pairs_nan_propagates():
    inp = workloads.forward_inputs(workloads.FWD_LONG_BF16.with_(B=2, T=1500, C=128, seed=33))
    inp["k"][0, 600, 3] = np.nan
    inp["v"][1, 900, 70] = np.nan
    y = host(run_forward(to_device(inp), "chunked", 0))
    assert np.all(np.isnan(y[0, 600:, 3])) and np.all(np.isnan(y[1, 900:, 70]))
    assert np.all(np.isfinite(y[0, :600, 3])) and np.all(np.isfinite(y[:, :, 71:]))


def test_bf16_odd_width():
    """bfloat16 with an odd C: no row pairs, one 2-byte channel per lane, at the default tile and
    the longest one, across a ragged last tile."""
    inp = workloads.forward_inputs(workloads.FWD_LONG_BF16.with_(B=2, T=1100, C=99, seed=99))
    check(inp, algos=[("seq", 0), ("chunked", 0), ("chunked", 512)])


def test_bf16_output_is_rounded_float32_output():
    """The bf16 path computes in float32 and rounds y to nearest-even once.

    The sequential walk does the same float32 operations for both dtypes, so its bf16
    output is bit for bit the rounded float32 output.  The chunked scan runs two
    channels per thread for bf16 (one for float32), which changes how many tokens a
    wave aggregates and so the float32 rounding: there each bf16 output must be the
    rounding of some float32 value within 1e-6 * s of the float32 path's output
    (s = the convex weights applied to |v|, the scale of the error metric)."""
    inp = workloads.forward_inputs(workloads.FWD_LONG_BF16.with_(T=600, C=192))
    _, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    dev = to_device(inp)
    dev32 = dict(dev, k=dev["k"].float(), v=dev["v"].float())
    for algo, cl in (("seq", 0), ("chunked", 128)):
        y16 = run_forward(dev, algo, cl).float().cpu().numpy()
        y32 = run_forward(dev32, algo, cl).cpu().numpy()
        if algo == "seq":
            assert np.array_equal(y16, round_to_bf16(y32)), algo
        else:
            d = 1e-6 * s_ref
            lo = round_to_bf16((y32 - d).astype(np.float32))
            hi = round_to_bf16((y32 + d).astype(np.float32))
            assert np.all((lo <= y16) & (y16 <= hi)), algo
            assert np.mean(y16 == round_to_bf16(y32)) >= 0.99, algo


def test_deterministic():
    inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=3, T=2000, C=200, k_std=2.0))
    dev = to_device(inp)
    for algo, cl in (("seq", 0), ("chunked", 64)):
        a = run_forward(dev, algo, cl)
        b = run_forward(dev, algo, cl)
        assert torch.equal(a, b), algo


def test_state_handoff_matches_single_pass():
    """forward(T1) -> state -> forward(T - T1 from state) equals forward(T) (constant-size state)."""
    inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=2, T=900, C=96, k_std=2.0, seed=3))
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    dev = to_device(inp)
    for algo, cl in (("seq", 0), ("chunked", 128)):
        first = dict(dev, k=dev["k"][:, :333].contiguous(), v=dev["v"][:, :333].contiguous())
        rest = dict(dev, k=dev["k"][:, 333:].contiguous(), v=dev["v"][:, 333:].contiguous())
        y1, st = run_forward(first, algo, cl, return_state=True)
        y2 = run_forward(rest, algo, cl, state=st)
        y = np.concatenate([host(y1), host(y2)], axis=1)
        assert scaled_error(y, y_ref, s_ref) <= TOL["f32"], algo


def test_final_state_matches_oracle():
    inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=2, T=500, C=80, k_std=2.0, seed=4))
    _, (a, b, p) = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_state=True)
    dev = to_device(inp)
    for algo, cl in (("seq", 0), ("chunked", 64), ("chunked", 256)):
        _, (ga, gb, gp) = run_forward(dev, algo, cl, return_state=True)
        ga, gb, gp = host(ga), host(gb), host(gp)
        np.testing.assert_allclose(gp + np.log(gb), p + np.log(b), rtol=0, atol=2e-5)
        np.testing.assert_allclose(ga / gb, a / b, rtol=0, atol=2e-5 * np.max(np.abs(inp["v"])))


# ---- invariants and special cases on the GPU ----

def special(B=2, T=400, C=70, seed=9, **kw):
    return workloads.forward_inputs(workloads.FWD_SMALL.with_(B=B, T=T, C=C, seed=seed, **kw))


def run_all(inp):
    dev = to_device(inp)
    return [(algo, cl, host(run_forward(dev, algo, cl))) for algo, cl in ALGOS]


def test_constant_v():
    inp = special(k_std=2.0)
    inp["v"][:] = np.float32(-1.25)
    for algo, cl, y in run_all(inp):
        np.testing.assert_allclose(y, -1.25, rtol=1e-5, err_msg=f"{algo} {cl}")


def test_single_token_gives_v():
    inp = special(T=1, C=300)
    for algo, cl, y in run_all(inp):
        np.testing.assert_allclose(y, inp["v"], rtol=1e-6, atol=0, err_msg=algo)


@pytest.mark.parametrize("shift", [200.0, -200.0])
def test_key_shift(shift):
    """k + 200 overflows a naive float32 exponential; the result must not change."""
    inp = special(k_std=2.0)
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    inp["k"] = (inp["k"].astype(np.float64) + shift).astype(np.float32)
    y_ref2, s_ref2 = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    assert scaled_error(y_ref2, y_ref, s_ref) < 1e-5  # the float32 rounding of k+shift itself
    for algo, cl, y in run_all(inp):
        assert scaled_error(y, y_ref2, s_ref2) <= TOL["f32"], (algo, cl)


def test_u_equal_w_large_gives_current_v():
    inp = special()
    inp["w"][:] = 60.0
    inp["u"][:] = 60.0
    for algo, cl, y in run_all(inp):
        np.testing.assert_allclose(y, inp["v"], rtol=1e-6, atol=1e-30, err_msg=algo)


def test_large_w_keeps_newest_past_token():
    inp = special()
    inp["w"][:] = 1000.0
    k = inp["k"].astype(np.float64)
    v = inp["v"].astype(np.float64)
    u = inp["u"].astype(np.float64)
    want = np.empty_like(v)
    want[:, 0] = v[:, 0]
    ep, ec = np.exp(k[:, :-1]), np.exp(u[None, None, :] + k[:, 1:])
    want[:, 1:] = (ep * v[:, :-1] + ec * v[:, 1:]) / (ep + ec)
    for algo, cl, y in run_all(inp):
        np.testing.assert_allclose(y, want, rtol=3e-6, atol=3e-6, err_msg=algo)


@pytest.mark.parametrize("case", ["negative_w", "huge_k_range", "huge_u", "tiny_u", "w_zero"])
def test_exact_fallback_cases(case):
    """Inputs outside the fast path's conditioning run the exact per-token path."""
    inp = special(T=300, C=130, seed=11)
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
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    for algo, cl, y in run_all(inp):
        assert scaled_error(y, y_ref, s_ref) <= TOL["f32"], (case, algo, cl)


def test_nan_propagates():
    inp = special(T=200, C=64)
    inp["k"][0, 50, 3] = np.nan
    inp["v"][1, 120, 7] = np.nan
    for algo, cl, y in run_all(inp):
        assert np.all(np.isnan(y[0, 50:, 3])), algo
        assert np.all(np.isnan(y[1, 120:, 7])), algo
        assert np.all(np.isfinite(y[0, :50, 3])) and np.all(np.isfinite(y[:, :, 8:])), algo


@pytest.mark.parametrize("C", [192, 130])
def test_long_sequences_every_tile(C):
    """Hundreds of chunks per channel group: the look-back folds long runs of published
    aggregates.  Repeated launches on one workspace must agree bit for bit and with the
    oracle on every element."""
    inp = workloads.forward_inputs(workloads.FWD_SMALL.with_(B=2, T=20000, C=C, k_std=1.5, seed=C))
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    dev = to_device(inp)
    k = dev["k"]
    for cl in (64, 128, 256):
        ws = libwkv.new_workspace(2, 20000, C, k.dtype, "chunked", cl)
        first = None
        for rep in range(3):
            y = libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo="chunked", chunk_len=cl,
                                   workspace=ws)
            torch.cuda.synchronize()
            assert libwkv.lookback_error(ws) == 0
            err = scaled_error(host(y), y_ref, s_ref)
            assert err <= TOL["f32"], (cl, rep, err)
            if first is None:
                first = y.clone()
            else:
                assert torch.equal(first, y), (cl, rep)


def test_workspace_epoch_counts_chunked_calls():
    """Each chunked call opens a new record epoch; a sequential call leaves it alone."""
    inp = special(B=1, T=700, C=64)
    dev = to_device(inp)
    k = dev["k"]
    ws = libwkv.new_workspace(1, 700, 64, k.dtype, "chunked", 128)
    assert libwkv.workspace_query(ws) == (0, 0)
    for n in range(1, 4):
        libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo="chunked", chunk_len=128, workspace=ws)
        assert libwkv.workspace_query(ws) == (0, n)
    libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo="seq", workspace=ws)
    assert libwkv.workspace_query(ws) == (0, 3)


@pytest.mark.parametrize("T", [900, 20000])
def test_stale_ticket_counter_is_flagged(T):
    """A workspace whose ticket counter was not zero (here: set past every tile) makes the chunked
    forward flag the call; every tile is still computed once (ticket mod the number of tiles, or
    the workgroup index, on the path that waits for nothing), so y matches the oracle, and the
    launch's last workgroup leaves the counters ready for the next call.  T = 900: 32 tiles, fewer
    than the compute units, numbered by workgroup index; T = 20000: 628 tiles, numbered by ticket."""
    inp = special(B=2, T=T, C=128)
    dev = to_device(inp)
    k = dev["k"]
    y_ref, s_ref = wkv_recurrent(inp["w"], inp["u"], inp["k"], inp["v"], return_scale=True)
    ws = libwkv.new_workspace(2, T, 128, k.dtype, "chunked", 128)
    ws.view(torch.int32)[0] = (1 << 30) + 5  # the ticket counter (first word of the control block)
    y = torch.full_like(k, 7.0)
    libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo="chunked", chunk_len=128, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 1
    assert scaled_error(host(y), y_ref, s_ref) <= TOL["f32"]
    y = libwkv.wkv_forward(dev["w"], dev["u"], k, dev["v"], algo="chunked", chunk_len=128, workspace=ws)
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 0
    assert scaled_error(host(y), y_ref, s_ref) <= TOL["f32"]
