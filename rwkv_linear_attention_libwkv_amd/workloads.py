"""Seeded synthetic inputs for the WKV workloads.

This module holds none of the operator's arithmetic.  It draws random numbers,
applies the distributions' parameters and rounds values to the storage dtype,
so that the libwkv binding and the float64 oracle receive exactly the same
inputs.  Stand-ins: the pages evaluate whole models on datasets (LAMBADA, PIQA,
the Pile); none of that reaches the operator, so these synthetic tensors have
the operator's shapes (channel widths of the 169M, 1.5B and 14B models the
pages name, contexts up to 64K tokens) and plain value distributions.

Conventions
-----------
* N(0, s) means mean 0 and *standard deviation* s; U(a, b) is uniform on [a, b).
* w = exp(w_raw) per channel (the decay rate itself, used as e^{-w}).
* One NumPy ``default_rng(seed)`` stream per forward workload, drawn in the
  order w_raw, u, k, v, each as one full draw.
* bf16 tensors are float32 samples rounded to nearest-even; the oracle sees the
  rounded values.
* Decode-step workloads draw per-step k, v with ``torch.Generator`` seeded by
  (seed, step) on the device that will hold them.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ForwardSpec:
    """A whole-sequence workload: k, v, y of shape [B, T, C]; w, u of shape [C]."""

    name: str
    B: int
    T: int
    C: int
    dtype: str  # "f32" or "bf16" (k, v, y); w, u are always float32
    k_std: float = 1.0
    v_std: float = 1.0
    w_raw_lo: float = -3.0
    w_raw_hi: float = 1.0
    u_std: float = 0.5
    seed: int = 0

    @property
    def elements(self) -> int:
        return self.B * self.T * self.C

    def with_(self, **kw) -> "ForwardSpec":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class StepSpec:
    """A batched decode workload: N sequences x G layer slots x C channels."""

    name: str
    N: int
    G: int
    C: int
    steps: int
    prefix: int
    dtype: str = "bf16"
    k_std: float = 1.0
    v_std: float = 1.0
    w_raw_lo: float = -3.0
    w_raw_hi: float = 1.0
    u_std: float = 0.5
    seed: int = 0

    @property
    def lanes(self) -> int:
        return self.N * self.G * self.C

    def with_(self, **kw) -> "StepSpec":
        return dataclasses.replace(self, **kw)


# The five workloads.  Widths stand in for the model sizes the pages name.
FWD_SMALL = ForwardSpec("wkv_fwd_f32_B1_T64_C64", 1, 64, 64, "f32")
FWD_169M = ForwardSpec("wkv_fwd_f32_B8_T1024_C768", 8, 1024, 768, "f32")
FWD_CTX8K = ForwardSpec(
    "wkv_fwd_f32_B8_T8192_C2048", 8, 8192, 2048, "f32",
    k_std=2.0, w_raw_lo=-5.0, w_raw_hi=1.0, u_std=1.0,
)
FWD_LONG_BF16 = ForwardSpec(
    "wkv_fwd_bf16_B1_T65536_C5120", 1, 65536, 5120, "bf16",
    w_raw_lo=-6.0, w_raw_hi=1.0, u_std=0.5,
)
STEP_DECODE = StepSpec("wkv_step_bf16_N256_G32_C4096_x16", 256, 32, 4096, steps=16, prefix=128)
# one sequence through the same 32 layer slots: launch-bound (4 MB per step)
STEP_DECODE_SMALL = StepSpec("wkv_step_bf16_N1_G32_C4096_x16", 1, 32, 4096, steps=16, prefix=16)

FORWARD_SPECS = {s.name: s for s in (FWD_SMALL, FWD_169M, FWD_CTX8K, FWD_LONG_BF16)}


@dataclass(frozen=True)
class LinearAttnSpec:
    """Causal linear attention: q, k [BH, N, D], v and the output [BH, N, M] (BH = batch x heads)."""

    name: str
    BH: int
    N: int
    D: int
    M: int
    dtype: str = "f32"
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.BH * self.N

    def with_(self, **kw) -> "LinearAttnSpec":
        return dataclasses.replace(self, **kw)


# Shapes of the linear-transformer page's experiments: 8 heads of 32 dimensions (embedding
# 256); MNIST generation (784 pixels, batch 10), CIFAR-10 generation (3072 values, batch 4),
# and the long-sequence scaling runs (up to 2^14 positions at which the baselines still ran).
LA_SMALL = LinearAttnSpec("la_f32_BH2_N300_D32_M32", 2, 300, 32, 32)
LA_MNIST = LinearAttnSpec("la_f32_BH80_N784_D32_M32", 80, 784, 32, 32)
LA_CIFAR = LinearAttnSpec("la_f32_BH32_N3072_D32_M32", 32, 3072, 32, 32)
LA_LONG = LinearAttnSpec("la_f32_BH64_N16384_D32_M32", 64, 16384, 32, 32)
LA_LONG_BF16 = LinearAttnSpec("la_bf16_BH64_N16384_D32_M32", 64, 16384, 32, 32, "bf16")
LA_SPECS = {s.name: s for s in (LA_SMALL, LA_MNIST, LA_CIFAR, LA_LONG, LA_LONG_BF16)}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def channel_params(rng, shape, w_raw_lo, w_raw_hi, u_std):
    """Draw (w, u) as float32: w = exp(U(lo, hi)), u = N(0, u_std)."""
    w_raw = rng.uniform(w_raw_lo, w_raw_hi, size=shape)
    u = rng.normal(0.0, u_std, size=shape)
    return np.exp(w_raw).astype(np.float32), u.astype(np.float32)


def forward_inputs(spec: ForwardSpec) -> dict:
    """Seeded inputs of a forward workload as NumPy float32 arrays.

    Returns {"w": [C], "u": [C], "k": [B,T,C], "v": [B,T,C], "dtype": ...};
    for bf16 workloads k and v already hold bf16-representable values.
    """
    rng = np.random.default_rng(spec.seed)
    w, u = channel_params(rng, (spec.C,), spec.w_raw_lo, spec.w_raw_hi, spec.u_std)
    shape = (spec.B, spec.T, spec.C)
    k = rng.standard_normal(size=shape, dtype=np.float32)
    k *= np.float32(spec.k_std)
    v = rng.standard_normal(size=shape, dtype=np.float32)
    v *= np.float32(spec.v_std)
    if spec.dtype == "bf16":
        k = round_to_bf16(k)
        v = round_to_bf16(v)
    elif spec.dtype != "f32":
        raise ValueError(f"unknown dtype {spec.dtype!r}")
    return {"w": w, "u": u, "k": k, "v": v, "dtype": spec.dtype}


def backward_inputs(spec: ForwardSpec) -> dict:
    """forward_inputs(spec) plus gy = dL/dy ~ N(0, 1) of shape [B, T, C].

    gy comes from its own stream, ``default_rng(seed + 7_777_777)``, so the forward
    inputs are those of the forward workload; bf16 workloads round it like k and v.
    """
    inp = forward_inputs(spec)
    rng = np.random.default_rng(spec.seed + 7_777_777)
    gy = rng.standard_normal(size=(spec.B, spec.T, spec.C), dtype=np.float32)
    inp["gy"] = round_to_bf16(gy) if spec.dtype == "bf16" else gy
    return inp


def linear_attention_inputs(spec: LinearAttnSpec) -> dict:
    """q, k, v ~ N(0, 1) as float32 (bf16-representable for bf16 workloads), drawn in that order
    from default_rng(seed)."""
    rng = np.random.default_rng(spec.seed)
    out = {"dtype": spec.dtype}
    for name, last in (("q", spec.D), ("k", spec.D), ("v", spec.M)):
        x = rng.standard_normal(size=(spec.BH, spec.N, last), dtype=np.float32)
        out[name] = round_to_bf16(x) if spec.dtype == "bf16" else x
    return out


def step_params(spec: StepSpec) -> tuple:
    """(w, u) of a decode workload, shape [G, C], float32."""
    rng = np.random.default_rng(spec.seed)
    return channel_params(rng, (spec.G, spec.C), spec.w_raw_lo, spec.w_raw_hi, spec.u_std)


def step_kv(spec: StepSpec, step: int, device="cpu"):
    """k, v of decode step ``step`` (prefix steps first) as torch tensors [N, G, C].

    Drawn with a torch.Generator on ``device`` seeded from (seed, step), then
    rounded to the workload dtype.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (spec.seed + 1) + step)
    shape = (spec.N, spec.G, spec.C)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * spec.k_std
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * spec.v_std
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    return k.to(tdt), v.to(tdt)


def sample_lanes(n_rows: int, n_cols: int, count: int, seed: int = 12345):
    """``count`` distinct (row, col) pairs, always including both corners."""
    rng = np.random.default_rng(seed)
    total = n_rows * n_cols
    count = min(count, total)
    flat = rng.choice(total, size=count, replace=False)
    flat[0] = 0
    if count > 1:
        flat[1] = total - 1
    flat = np.unique(flat)
    return [(int(f // n_cols), int(f % n_cols)) for f in flat]
