"""Seeded synthetic workloads for the selective scan and the SSD form.

This module only draws numbers: it holds no step of the scan.  Both the HIP
path and the fp64 oracle consume exactly the tensors produced here (cast once
to the workload's storage dtype, then widened exactly by the oracle).

Generator: numpy PCG64 (`default_rng(seed)`), drawn in float32 in a fixed
order so that a given (workload, seed, shape) is reproducible byte for byte:
  S6  : u, delta_raw, B, C, z, Dskip, delta_bias, spike positions
  SSD : X, delta_raw, B, C, A
  decode step : state, u, delta_raw, B, C, z, Dskip, delta_bias
  conv1d      : x, weight, bias
bf16 tensors are produced from float32 by torch's round-to-nearest-even cast.

Parameterisation conventions (stated on the pages, not part of the kernel):
A is the continuous-time diagonal, A = -exp(A_log) (negative so every
exp(delta*A) is a contraction); with A_log[d, n] = log(n + 1) this is
-(n + 1) after rounding to float32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class S6Workload:
    name: str
    B: int
    L: int
    D: int
    N: int
    dtype: str                    # storage dtype of u/delta/B/C/z/y: "f32" | "bf16"
    delta_mean: float             # delta_raw ~ N(delta_mean, delta_std)
    delta_std: float
    bias_range: Optional[tuple]   # delta_bias ~ U(lo, hi) or None
    skip: Optional[str]           # "ones" | "normal" (N(1, 0.1)) | None
    gate: bool                    # silu(z) gate with z ~ N(0, 1)
    spike_frac: float = 0.0       # fraction of token positions with delta_raw = +3
    a_from_log: bool = False      # A = -exp(log(n + 1)) vs A = -(n + 1) directly
    desc: str = ""

    def scaled(self, **kw) -> "S6Workload":
        return dataclasses.replace(self, **kw)

    @property
    def tok_ch(self) -> int:
        return self.B * self.L * self.D


@dataclasses.dataclass(frozen=True)
class SSDWorkload:
    name: str
    B: int
    L: int
    H: int
    P: int
    N: int
    G: int
    chunk: int
    dtype: str
    delta_mean: float = -2.0
    delta_std: float = 0.5
    desc: str = ""

    def scaled(self, **kw) -> "SSDWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def tok_ch(self) -> int:
        return self.B * self.L * self.H * self.P


@dataclasses.dataclass(frozen=True)
class StepWorkload:
    """One decode step of B sequences against a resident [B, D, N] state."""
    name: str
    B: int
    D: int
    N: int
    dtype: str
    desc: str = ""

    def scaled(self, **kw) -> "StepWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    """Causal depthwise conv1d + SiLU over [B, L, D] inputs, width K."""
    name: str
    B: int
    L: int
    D: int
    K: int
    dtype: str
    desc: str = ""

    def scaled(self, **kw) -> "ConvWorkload":
        return dataclasses.replace(self, **kw)


S6_SMALL_FP32 = S6Workload(
    "s6_small_fp32", B=1, L=256, D=64, N=16, dtype="f32", delta_mean=-2.0,
    delta_std=0.5, bias_range=None, skip="ones", gate=False,
    desc="S6 fp32, B=1 L=256 D=64 N=16, softplus(N(-2,0.5)), A=-(n+1), D=1")
S6_MAMBA130M = S6Workload(
    "s6_mamba130m_layer_bf16", B=8, L=2048, D=1536, N=16, dtype="bf16",
    delta_mean=0.0, delta_std=1.0, bias_range=(-4.0, -2.0), skip="normal",
    gate=True, a_from_log=True,
    desc="Mamba-130M-shaped layer scan, B=8 L=2048 D=1536 N=16, bf16 I/O, fp32 state")
S6_MAMBA2P8B = S6Workload(
    "s6_mamba2.8b_layer_bf16", B=4, L=4096, D=5120, N=16, dtype="bf16",
    delta_mean=0.0, delta_std=1.0, bias_range=(-4.0, -2.0), skip="normal",
    gate=True, a_from_log=True,
    desc="Mamba-2.8B-shaped layer scan, B=4 L=4096 D=5120 N=16, bf16 I/O, fp32 state")
S6_LONG_FP32 = S6Workload(
    "s6_long_fp32", B=1, L=131072, D=2048, N=16, dtype="f32", delta_mean=-4.0,
    delta_std=0.5, bias_range=None, skip=None, gate=False, spike_frac=0.01,
    desc="long-sequence scan, B=1 L=131072 D=2048 N=16 fp32, 1% delta spikes to +3")
SSD_MAMBA2 = SSDWorkload(
    "ssd_mamba2_bf16", B=4, L=8192, H=64, P=64, N=128, G=1, chunk=256,
    dtype="bf16", desc="Mamba-2 SSD, B=4 L=8192 H=64 P=64 N=128 G=1 chunk 256, bf16")

S6_DECODE_2P8B = StepWorkload(
    "s6_decode_mamba2.8b_bf16", B=64, D=5120, N=16, dtype="bf16",
    desc="decode step of 64 sequences through a Mamba-2.8B-shaped layer, D=5120 N=16, "
         "bf16 activations, fp32 state")

CONV_MAMBA130M = ConvWorkload(
    "conv1d_mamba130m_layer_bf16", B=8, L=2048, D=1536, K=4, dtype="bf16",
    desc="conv1d (d_conv=4) + SiLU in front of a Mamba-130M-shaped scan, B=8 L=2048 D=1536, bf16")

S6_WORKLOADS = {w.name: w for w in (S6_SMALL_FP32, S6_MAMBA130M, S6_MAMBA2P8B, S6_LONG_FP32)}
SSD_WORKLOADS = {w.name: w for w in (SSD_MAMBA2,)}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(dtype))


def make_s6_inputs(w: S6Workload, seed: int = 0) -> dict:
    """Tensors on the CPU for one S6 call: u, delta, A, B, C, D, z, delta_bias,
    h0 (None) and the flag delta_softplus (always on for these workloads)."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    shape = (w.B, w.L, w.D)
    u = rng.standard_normal(shape, dtype=f32)
    delta = rng.standard_normal(shape, dtype=f32)
    delta *= f32(w.delta_std)
    delta += f32(w.delta_mean)
    Bm = rng.standard_normal((w.B, w.L, w.N), dtype=f32)
    Cm = rng.standard_normal((w.B, w.L, w.N), dtype=f32)
    z = rng.standard_normal(shape, dtype=f32) if w.gate else None
    if w.skip == "ones":
        Dskip = np.ones(w.D, dtype=f32)
    elif w.skip == "normal":
        Dskip = (1.0 + 0.1 * rng.standard_normal(w.D)).astype(f32)
    else:
        Dskip = None
    bias = None
    if w.bias_range is not None:
        lo, hi = w.bias_range
        bias = rng.uniform(lo, hi, size=w.D).astype(f32)
    if w.spike_frac > 0:
        k = int(math.floor(w.spike_frac * w.L))
        pos = rng.choice(w.L, size=k, replace=False)
        delta[:, pos, :] = f32(3.0)
    n1 = np.arange(1, w.N + 1, dtype=np.float64)
    if w.a_from_log:
        A = -np.exp(np.log(n1))
    else:
        A = -n1
    A = np.broadcast_to(A, (w.D, w.N)).astype(f32)
    return dict(
        u=_cast(u, w.dtype), delta=_cast(delta, w.dtype),
        A=torch.from_numpy(np.ascontiguousarray(A)),
        B=_cast(Bm, w.dtype), C=_cast(Cm, w.dtype),
        D=None if Dskip is None else torch.from_numpy(Dskip),
        z=None if z is None else _cast(z, w.dtype),
        delta_bias=None if bias is None else torch.from_numpy(bias),
        h0=None, delta_softplus=True)


def make_ssd_inputs(w: SSDWorkload, seed: int = 0) -> dict:
    """Tensors on the CPU for one SSD call: X, delta, A [H], B, C, and no
    skip/gate/bias (the workload names none)."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    s = f32(1.0 / math.sqrt(w.N))
    X = rng.standard_normal((w.B, w.L, w.H, w.P), dtype=f32) * s
    delta = rng.standard_normal((w.B, w.L, w.H), dtype=f32)
    delta *= f32(w.delta_std)
    delta += f32(w.delta_mean)
    Bm = rng.standard_normal((w.B, w.L, w.G, w.N), dtype=f32) * s
    Cm = rng.standard_normal((w.B, w.L, w.G, w.N), dtype=f32) * s
    A = (-np.exp(rng.uniform(0.0, 2.0, size=w.H))).astype(f32)
    return dict(
        X=_cast(X, w.dtype), delta=_cast(delta, w.dtype),
        A=torch.from_numpy(A), B=_cast(Bm, w.dtype), C=_cast(Cm, w.dtype),
        D=None, z=None, delta_bias=None, h0=None, delta_softplus=True,
        chunk=w.chunk)


def make_step_inputs(w: StepWorkload, seed: int = 0) -> dict:
    """Tensors on the CPU for one decode step: state [B, D, N] fp32 ~ N(0, 1)
    (a state left by earlier tokens), u, delta_raw ~ N(0, 1), B, C, z ~ N(0, 1),
    Dskip ~ N(1, 0.1), delta_bias ~ U(-4, -2), A = -exp(log(n + 1)); softplus on."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    state = rng.standard_normal((w.B, w.D, w.N), dtype=f32)
    u = rng.standard_normal((w.B, w.D), dtype=f32)
    delta = rng.standard_normal((w.B, w.D), dtype=f32)
    Bm = rng.standard_normal((w.B, w.N), dtype=f32)
    Cm = rng.standard_normal((w.B, w.N), dtype=f32)
    z = rng.standard_normal((w.B, w.D), dtype=f32)
    Dskip = (1.0 + 0.1 * rng.standard_normal(w.D)).astype(f32)
    bias = rng.uniform(-4.0, -2.0, size=w.D).astype(f32)
    A = np.broadcast_to(-np.exp(np.log(np.arange(1, w.N + 1, dtype=np.float64))),
                        (w.D, w.N)).astype(f32)
    return dict(
        state=torch.from_numpy(state), u=_cast(u, w.dtype), delta=_cast(delta, w.dtype),
        A=torch.from_numpy(np.ascontiguousarray(A)), B=_cast(Bm, w.dtype), C=_cast(Cm, w.dtype),
        D=torch.from_numpy(Dskip), z=_cast(z, w.dtype), delta_bias=torch.from_numpy(bias),
        delta_softplus=True)


def make_conv_inputs(w: ConvWorkload, seed: int = 0) -> dict:
    """x ~ N(0, 1); weight, bias ~ U(-1/sqrt(K), 1/sqrt(K)) (the usual fan-in
    bound of a depthwise convolution with K taps)."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    x = rng.standard_normal((w.B, w.L, w.D), dtype=f32)
    bound = 1.0 / math.sqrt(w.K)
    weight = rng.uniform(-bound, bound, size=(w.D, w.K)).astype(f32)
    bias = rng.uniform(-bound, bound, size=w.D).astype(f32)
    return dict(x=_cast(x, w.dtype), weight=torch.from_numpy(weight), bias=torch.from_numpy(bias))


def conv_algorithmic_bytes(w: ConvWorkload) -> int:
    """x read once, u written once, weight and bias read once."""
    e = 4 if w.dtype == "f32" else 2
    return 2 * w.B * w.L * w.D * e + w.D * (w.K + 1) * 4


def step_algorithmic_bytes(w: StepWorkload) -> int:
    """State read and written once; A, u, delta, z, B, C, Dskip, bias read once; y written."""
    e = 4 if w.dtype == "f32" else 2
    n = 2 * w.B * w.D * w.N * 4          # state in and out
    n += w.D * w.N * 4                   # A
    n += 4 * w.B * w.D * e               # u, delta, z, y
    n += 2 * w.B * w.N * e               # B, C
    n += 2 * w.D * 4                     # Dskip, delta_bias
    return n


def s6_algorithmic_bytes(w: S6Workload, with_h_last: bool = True) -> int:
    """Every input read once, y and the final state written once."""
    e = 4 if w.dtype == "f32" else 2
    tok = w.B * w.L * w.D
    n = 2 * tok * e                                   # u, delta
    n += 2 * w.B * w.L * w.N * e                      # B, C
    n += w.D * w.N * 4                                # A
    if w.gate:
        n += tok * e                                  # z
    if w.skip:
        n += w.D * 4
    if w.bias_range is not None:
        n += w.D * 4
    n += tok * e                                      # y
    if with_h_last:
        n += w.B * w.D * w.N * 4                      # final state
    return n


def ssd_algorithmic_bytes(w: SSDWorkload, with_h_last: bool = True) -> int:
    e = 4 if w.dtype == "f32" else 2
    tok = w.B * w.L * w.H * w.P
    n = 2 * tok * e                                   # X in, Y out
    n += w.B * w.L * w.H * e                          # delta
    n += 2 * w.B * w.L * w.G * w.N * e                # B, C
    n += w.H * 4                                      # A
    if with_h_last:
        n += w.B * w.H * w.P * w.N * 4
    return n
