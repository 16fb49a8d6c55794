"""Seeded synthetic inputs for the conv2d training layer (shared by tests, bench and smoke).

This module holds the workload table and the random draws only.  It contains none of
the layer's arithmetic: no convolution, no normalisation, no activation.  Both the fp64
oracle (``oracle/``) and the HIP library (``convolution_layer_amd``) are fed the arrays
it returns, so the two sides see bit-identical inputs.

Generator: ``numpy.random.default_rng(seed)`` (PCG64), fp64 draws in the fixed order
x, w, b, gamma, beta, dY (absent tensors are skipped).  Draws are rounded to the storage
dtype (fp32, or bf16 with round-to-nearest-even) before anyone sees them; the arrays
returned are float64 holding exactly those rounded values.

Layouts: x NHWC [N,H,W,IC]; w OHWI [OC,KH,KW,IC]; dY/z NHWC [N,OH,OW,OC].

Distribution notation N(m, s) means mean m and *standard deviation* s.  "He-normal"
means N(0, sqrt(2/fan_in)) with fan_in = KH*KW*IC.  Kaiming-uniform bounds follow the
weight initialiser of the rl_tools conv2d generic listing (``init_weights``): weight bound
sqrt(6/fan_in), bias bound 1/sqrt(fan_in).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

F32 = "f32"
BF16 = "bf16"

ACT_IDENTITY, ACT_RELU, ACT_TANH, ACT_SIGMOID, ACT_GELU = 0, 1, 2, 3, 4
NORM_NONE, NORM_BATCH, NORM_LAYER, NORM_GROUP = 0, 1, 2, 3


@dataclass(frozen=True)
class ConvShape:
    N: int
    H: int
    W: int
    IC: int
    OC: int
    KH: int
    KW: int
    sh: int = 1
    sw: int = 1
    ph: int = 0
    pw: int = 0

    @property
    def OH(self) -> int:
        return (self.H + 2 * self.ph - self.KH) // self.sh + 1

    @property
    def OW(self) -> int:
        return (self.W + 2 * self.pw - self.KW) // self.sw + 1

    @property
    def P(self) -> int:
        return self.N * self.OH * self.OW

    @property
    def Kdim(self) -> int:
        return self.KH * self.KW * self.IC

    @property
    def x_shape(self):
        return (self.N, self.H, self.W, self.IC)

    @property
    def w_shape(self):
        return (self.OC, self.KH, self.KW, self.IC)

    @property
    def y_shape(self):
        return (self.N, self.OH, self.OW, self.OC)

    def flops(self) -> int:
        """2*P*OC*Kdim: one multiply-add per (output, tap), padded taps counted."""
        return 2 * self.P * self.OC * self.Kdim

    def with_batch(self, n: int) -> "ConvShape":
        return replace(self, N=n)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ConvShape
    dtype: str
    act: int
    norm: int
    seed: int
    x_dist: tuple
    w_dist: tuple
    b_dist: tuple | None  # None: no bias pointer
    dy_dist: tuple
    gamma_dist: tuple | None = None
    beta_dist: tuple | None = None
    momentum: float = 0.1
    eps: float = 1e-5
    note: str = ""
    extra: dict = field(default_factory=dict)

    def with_batch(self, n: int) -> "Workload":
        return replace(self, shape=self.shape.with_batch(n))


def _he(fan):
    return ("normal", 0.0, math.sqrt(2.0 / fan))


def _ku_w(fan):
    b = math.sqrt(6.0 / fan)
    return ("uniform", -b, b)


def _ku_b(fan):
    b = 1.0 / math.sqrt(fan)
    return ("uniform", -b, b)


WORKLOADS: dict[str, Workload] = {}


def _add(w: Workload):
    WORKLOADS[w.name] = w


# 1: tiny fp32 layer, bias + ReLU, no norm.
_add(Workload("c1", ConvShape(4, 16, 16, 3, 8, 3, 3, 1, 1, 1, 1), F32, ACT_RELU, NORM_NONE, 1,
              ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), _ku_b(27), ("normal", 0.0, 1.0),
              note="tiny conv2d fp32 NHWC 16x16x3 -> 8, 3x3 s1 p1, bias, ReLU"))
# 2a/2b/2c: RL-encoder stack fp32, pad 0, ReLU, He-normal weights, zero bias.
_add(Workload("c2a", ConvShape(256, 84, 84, 4, 32, 8, 8, 4, 4, 0, 0), F32, ACT_RELU, NORM_NONE, 2,
              ("uniform", 0.0, 1.0), _he(256), ("zeros",), ("normal", 0.0, 1.0),
              note="RL encoder layer 1: 84x84x4 -> 20x20x32, 8x8 s4"))
_add(Workload("c2b", ConvShape(256, 20, 20, 32, 64, 4, 4, 2, 2, 0, 0), F32, ACT_RELU, NORM_NONE, 2,
              ("chain", "c2a"), _he(512), ("zeros",), ("normal", 0.0, 1.0),
              note="RL encoder layer 2: 20x20x32 -> 9x9x64, 4x4 s2 (input = layer-1 output)"))
_add(Workload("c2c", ConvShape(256, 9, 9, 64, 64, 3, 3, 1, 1, 0, 0), F32, ACT_RELU, NORM_NONE, 2,
              ("chain", "c2b"), _he(576), ("zeros",), ("normal", 0.0, 1.0),
              note="RL encoder layer 3: 9x9x64 -> 7x7x64, 3x3 s1"))
# 3: conv + batch-norm training layer fp32.
_add(Workload("c3", ConvShape(128, 32, 32, 64, 64, 3, 3, 1, 1, 1, 1), F32, ACT_RELU, NORM_BATCH, 3,
              ("normal", 0.0, 1.0), _ku_w(576), _ku_b(576), ("normal", 0.0, 1.0),
              gamma_dist=("uniform", 0.5, 1.5), beta_dist=("normal", 0.0, 0.1),
              note="conv + BatchNorm(train) + ReLU fp32, 32x32x64 -> 64"))
# 4: wide bf16 conv, fp32 accumulate, bias + tanh.
_add(Workload("c4", ConvShape(64, 56, 56, 128, 128, 3, 3, 1, 1, 1, 1), BF16, ACT_TANH, NORM_NONE, 4,
              ("normal", 0.0, 1.0), _he(1152), _ku_b(1152), ("normal", 0.0, 0.01),
              note="wide conv bf16 56x56x128 -> 128, 3x3 s1 p1, bias + tanh"))
# 5: weight-gradient-heavy bf16, no bias, identity.
_add(Workload("c5", ConvShape(8, 224, 224, 64, 64, 3, 3, 1, 1, 1, 1), BF16, ACT_IDENTITY, NORM_NONE, 5,
              ("normal", 0.0, 1.0), _he(576), None, ("normal", 0.0, 1.0),
              note="dW-heavy bf16 224x224x64 -> 64, 3x3 s1 p1, no bias, identity"))

RL_STACK = ("c2a", "c2b", "c2c")


def round_to(dtype: str, a) -> np.ndarray:
    """Round fp64 values to the storage dtype (RNE) and return them widened to fp64."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == F32:
        return a.astype(np.float32).astype(np.float64)
    if dtype == BF16:
        import torch
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float64).numpy()
    raise ValueError(dtype)


def _draw(rng: np.random.Generator, dist, shape) -> np.ndarray:
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size=shape)
    if kind == "zeros":
        return np.zeros(shape)
    raise ValueError(dist)


def make_inputs(wl: Workload, rng: np.random.Generator | None = None) -> dict:
    """Draw x, w, b, gamma, beta, dY for one workload.

    Returns float64 arrays holding values already rounded to the storage dtype (bias,
    gamma, beta, running stats are fp32 whatever the data dtype).  For a chained layer
    (x_dist ``("chain", ...)``) no x is drawn: the caller supplies the previous layer's
    output.  Pass ``rng`` to continue a shared stream (the RL stack shares seed 2).
    """
    s = wl.shape
    if rng is None:
        rng = np.random.default_rng(wl.seed)
    out = {}
    if wl.x_dist[0] != "chain":
        out["x"] = round_to(wl.dtype, _draw(rng, wl.x_dist, s.x_shape))
    out["w"] = round_to(wl.dtype, _draw(rng, wl.w_dist, s.w_shape))
    if wl.b_dist is not None:
        out["b"] = round_to(F32, _draw(rng, wl.b_dist, (s.OC,)))
    if wl.norm == NORM_BATCH:
        out["gamma"] = round_to(F32, _draw(rng, wl.gamma_dist, (s.OC,)))
        out["beta"] = round_to(F32, _draw(rng, wl.beta_dist, (s.OC,)))
        out["running_mean"] = np.zeros(s.OC)
        out["running_var"] = np.ones(s.OC)
    out["dy"] = round_to(wl.dtype, _draw(rng, wl.dy_dist, s.y_shape))
    return out


def synthetic_preactivation(wl: Workload, seed: int | None = None) -> np.ndarray:
    """A stand-in for a conv output z [N,OH,OW,OC] with per-channel structure.

    z[..., c] = m_c + s_c * N(0,1), m_c ~ U(-0.5, 0.5), s_c ~ U(0.5, 2.0).  Used where a
    call is tested on its own at full size (batch-norm statistics, activation backward)
    and computing z by the oracle's full convolution would take too long.
    """
    s = wl.shape
    rng = np.random.default_rng(1000 + wl.seed if seed is None else seed)
    m = rng.uniform(-0.5, 0.5, size=(s.OC,))
    sd = rng.uniform(0.5, 2.0, size=(s.OC,))
    z = m + sd * rng.standard_normal(size=s.y_shape)
    return round_to(wl.dtype, z)


def synthetic_grad(wl: Workload, scale: float = 1.0, seed: int | None = None) -> np.ndarray:
    """A stand-in gradient dZ [N,OH,OW,OC] ~ N(0, scale), rounded to the data dtype."""
    s = wl.shape
    rng = np.random.default_rng(2000 + wl.seed if seed is None else seed)
    return round_to(wl.dtype, scale * rng.standard_normal(size=s.y_shape))


def random_tensor(shape, dtype: str, seed: int, dist=("normal", 0.0, 1.0)) -> np.ndarray:
    """Generic seeded tensor for shape sweeps in the tests."""
    rng = np.random.default_rng(seed)
    return round_to(dtype, _draw(rng, dist, shape))


def device_normal(shape, dtype: str, seed: int, std: float = 1.0):
    """Seeded N(0, std) tensor drawn directly on the GPU (torch's CUDA Philox generator),
    rounded to the data dtype: for shapes too large to draw on the host.  Tests hand the
    oracle host copies of small windows of it."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std
    return t.to(torch.bfloat16 if dtype == BF16 else torch.float32)
