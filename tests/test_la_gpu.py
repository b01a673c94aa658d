"""GPU parity of wkv_linear_attention against the float64 oracle.

Gate: scale-normalised error |out - ref| / s, with s the same normalised average applied to
|v| (s >= |out|).  float32 (float32 matrix cores): 5e-5 -- every output is a ratio of sums of
positive weights, each accumulated in float32 over at most 32 products per tile step plus one
addition per sub-chunk and per chunk of the carried state.  bfloat16: 1e-2 -- phi, the
masked similarities and the carried state enter the bf16 matrix cores rounded to bf16 (2^-9
each) and the output is rounded once.
"""
import numpy as np
import pytest
import torch

from oracle import scaled_error
from oracle.linear_attention import elu_feature, linear_attention_direct, linear_attention_recurrent
from rwkv_linear_attention_libwkv_amd import libwkv, workloads
from tests.gpu_util import TORCH_DT, host

pytestmark = pytest.mark.gpu

TOL = {"f32": 5e-5, "bf16": 1e-2}


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(TORCH_DT[dtype])


ALGOS = ["one", "three"]


def run(inp, feature=True, algo="auto"):
    d = inp["dtype"]
    q, k, v = dev(inp["q"], d), dev(inp["k"], d), dev(inp["v"], d)
    ws = libwkv.new_la_workspace(*q.shape, v.shape[2], q.dtype)
    out = host(libwkv.linear_attention(q, k, v, feature_map=feature, workspace=ws, algo=algo))
    assert libwkv.lookback_error(ws) == 0
    return out


def check(spec, feature=True, label="", algo="auto"):
    inp = workloads.linear_attention_inputs(spec)
    if not feature:  # positive features given directly
        inp["q"] = np.float32(elu_feature(inp["q"]))
        inp["k"] = np.float32(elu_feature(inp["k"]))
        if spec.dtype == "bf16":
            inp["q"] = workloads.round_to_bf16(inp["q"])
            inp["k"] = workloads.round_to_bf16(inp["k"])
    out = run(inp, feature, algo)
    ref, scale = linear_attention_direct(inp["q"], inp["k"], inp["v"], feature=feature, return_scale=True)
    err = scaled_error(out, ref, scale)
    print(f"  {label} {spec.name} BH={spec.BH} N={spec.N} D={spec.D} feature={feature} {algo}: {err:.2e}", flush=True)
    assert err <= TOL[spec.dtype], err


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("feature", [True, False])
def test_small(dtype, feature, algo):
    check(workloads.LA_SMALL.with_(dtype=dtype, seed=1), feature, algo=algo)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 255, 256, 257, 511, 512, 513, 600, 1100])
def test_ragged_lengths(dtype, N, algo):
    check(workloads.LA_SMALL.with_(BH=3, N=N, dtype=dtype, seed=N), label="ragged", algo=algo)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_dim_64(dtype, algo):
    check(workloads.LA_SMALL.with_(BH=2, N=700, D=64, M=64, dtype=dtype, seed=7), label="D=64", algo=algo)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,M", [(32, 64), (64, 32)])
@pytest.mark.parametrize("N", [257, 700])
def test_feature_and_value_widths_differ(dtype, D, M, N, algo):
    """q, k of D features and v of M values with D != M (chunks of 256 positions)."""
    spec = workloads.LA_SMALL.with_(BH=3, N=N, D=D, M=M, dtype=dtype, seed=D + M + N)
    check(spec, label=f"D={D} M={M}", algo=algo)
    check(spec, feature=False, label=f"D={D} M={M}", algo=algo)
    inp = workloads.linear_attention_inputs(spec)
    assert np.array_equal(run(inp, algo="one"), run(inp, algo="three"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64])
def test_evaluations_agree_bitwise(dtype, D):
    """The one-pass and three-launch evaluations add the same floats in the same order."""
    spec = workloads.LA_SMALL.with_(BH=5, N=1500, D=D, M=D, dtype=dtype, seed=3)
    inp = workloads.linear_attention_inputs(spec)
    one, three = run(inp, algo="one"), run(inp, algo="three")
    assert np.array_equal(one, three)


def test_mnist_shape():
    """BH = 80 (batch 10 x 8 heads), N = 784, D = M = 32, float32: every output."""
    check(workloads.LA_MNIST, label="mnist")


def test_long_sequences_sampled():
    """BH = 64, N = 16384: sampled sequences, every output against the cumulative-state oracle
    with its per-element scale (the same normalised sum applied to |v|)."""
    for spec in (workloads.LA_LONG, workloads.LA_LONG_BF16):
        inp = workloads.linear_attention_inputs(spec)
        out = run(inp)
        for b in (0, 37, spec.BH - 1):
            sl = {n: inp[n][b:b + 1] for n in ("q", "k", "v")}
            ref, scale = linear_attention_recurrent(sl["q"], sl["k"], sl["v"], return_scale=True)
            err = scaled_error(out[b:b + 1], ref, scale)
            print(f"  {spec.name} seq {b}: {err:.2e}", flush=True)
            assert err <= TOL[spec.dtype], err


def test_deterministic():
    """Fresh workspaces and one workspace reused by successive calls give the same bits."""
    spec = workloads.LA_CIFAR.with_(BH=8)
    inp = workloads.linear_attention_inputs(spec)
    q, k, v = (dev(inp[n], "f32") for n in ("q", "k", "v"))
    a = libwkv.linear_attention(q, k, v)
    b = libwkv.linear_attention(q, k, v)
    ws = libwkv.new_la_workspace(spec.BH, spec.N, spec.D, spec.M, q.dtype)
    order = ["one", "three", "one", "one", "auto"]  # the three-launch path leaves the counter alone
    reused = [libwkv.linear_attention(q, k, v, workspace=ws, algo=al).clone() for al in order]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for c in reused:
        assert torch.equal(a, c)
    assert libwkv.lookback_error(ws) == 0 and libwkv.workspace_epoch(ws) >= 3


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_long_sequence(dtype, algo):
    """BH = 1, N = 16384: 32 chunks chained through one sequence's look-backs, every output
    against the cumulative-state oracle with its per-element scale."""
    spec = workloads.LA_LONG.with_(BH=1, dtype=dtype, seed=11)
    inp = workloads.linear_attention_inputs(spec)
    out = run(inp, algo=algo)
    ref, scale = linear_attention_recurrent(inp["q"], inp["k"], inp["v"], return_scale=True)
    err = scaled_error(out, ref, scale)
    print(f"  one sequence N={spec.N} {dtype} {algo}: {err:.2e}", flush=True)
    assert err <= TOL[dtype]


def test_stale_ticket_counter_is_flagged():
    """The one-pass evaluation with a ticket counter that was not zero (here: past every chunk)
    flags the call; every chunk is still computed once (ticket mod the number of chunks, on the
    path that waits for nothing), so the outputs match the oracle, and the next call on the
    workspace is back on the usual path."""
    spec = workloads.LA_SMALL.with_(BH=3, N=700, seed=5)
    inp = workloads.linear_attention_inputs(spec)
    q, k, v = (dev(inp[n], "f32") for n in ("q", "k", "v"))
    ref, scale = linear_attention_direct(inp["q"], inp["k"], inp["v"], return_scale=True)
    ws = libwkv.new_la_workspace(spec.BH, spec.N, spec.D, spec.M, q.dtype)
    ws.view(torch.int32)[0] = (1 << 30) + 3  # the ticket counter (first word of the control block)
    out = torch.full_like(v, 7.0)
    libwkv.linear_attention(q, k, v, out=out, workspace=ws, algo="one")
    torch.cuda.synchronize()
    assert libwkv.lookback_error(ws) == 1
    assert scaled_error(host(out), ref, scale) <= TOL["f32"]
    out = host(libwkv.linear_attention(q, k, v, workspace=ws, algo="one"))
    assert libwkv.lookback_error(ws) == 0
    assert scaled_error(out, ref, scale) <= TOL["f32"]
