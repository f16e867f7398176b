"""Seeded synthetic workloads for the ParaRNN hot path.

This module only draws random inputs; it holds none of the method's
arithmetic.  It is the one piece of code that both the GPU path's tests and
the CPU oracle consume: the same bytes go to both sides.

Every stream comes from ``numpy.random.Generator(PCG64(seed))`` in a fixed
draw order.  Pre-activations are drawn in float32; bf16 workloads round them
to nearest-even bf16 once, here, and both sides read those same bits.

Workloads (the five benchmark shapes of this project):
  0  diag GRU   fp32   B=1  T=256     D=16    K=3
  1  linear     fp32   B=8  T=16384   D=1024  one scan (exact)
  2  diag GRU   bf16   B=2  T=4096    D=4096  K=3
  3  diag LSTM  fp32   B=4  T=8192    D=2048  K=3
  4  diag GRU   bf16   B=1  T=131072  D=1024  tol 1e-5, <= 8 iterations, + VJP
Distributions: U ~ N(0,1); recurrent weights ~ U(-0.5, 0.5); biases
~ N(0, 0.1^2) (0.1 is the standard deviation); LSTM forget bias = +1.0;
linear scan a_t = sigmoid(z), z ~ N(0,1), b_t ~ N(0,1); upstream gradient
dL/dh ~ N(0,1) fp32.  Head-wise block GRU (head size hs): each dense
recurrent block ~ U(-1/sqrt(hs), 1/sqrt(hs)) (torch's default recurrent
initialisation for a hidden size of hs), other draws as for the GRU.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GATES = {"linear": 2, "gru": 3, "lstm": 4, "slstm": 4, "head_gru": 3}
STATE = {"linear": 1, "gru": 1, "lstm": 2, "slstm": 4, "head_gru": 1}


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    cell: str
    B: int
    T: int
    D: int
    dtype: str          # storage dtype of the pre-activations: "f32" | "bf16"
    max_iters: int
    tol: float = 0.0    # > 0: stop on max residual < tol
    vjp: bool = False

    @property
    def N(self) -> int:
        return self.B * self.T * self.D


WORKLOADS = [
    Workload(0, "diag-gru-f32-B1-T256-D16-K3", "gru", 1, 256, 16, "f32", 3),
    Workload(1, "linear-scan-f32-B8-T16384-D1024", "linear", 8, 16384, 1024, "f32", 1),
    Workload(2, "diag-gru-bf16-B2-T4096-D4096-K3", "gru", 2, 4096, 4096, "bf16", 3),
    Workload(3, "diag-lstm-f32-B4-T8192-D2048-K3", "lstm", 4, 8192, 2048, "f32", 3),
    Workload(4, "diag-gru-bf16-B1-T131072-D1024-tol1e-5-vjp", "gru", 1, 131072, 1024, "bf16", 8, 1e-5, True),
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    cell: str
    B: int
    T: int
    D: int
    dtype: str
    pre: list = field(default_factory=list)   # G planes [B][T][D]: float32, or uint16 bf16 bits
    w: np.ndarray | None = None               # [G][D] float32
    bias: np.ndarray | None = None            # [G][D] float32
    g: np.ndarray | None = None               # [B][T][D] float32 upstream gradient (VJP)
    head_size: int = 1                        # head_gru: channels per head; w is [3][D/hs][hs][hs]

    @property
    def G(self):
        return GATES[self.cell]

    @property
    def S(self):
        return STATE[self.cell]

    def pre_f32(self):
        """The pre-activations as float32 values (bf16 widened exactly)."""
        if self.dtype == "bf16":
            return [bf16_bits_to_f32(p) for p in self.pre]
        return list(self.pre)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _uniform_half(rng, shape):
    return (rng.random(size=shape, dtype=np.float32) - np.float32(0.5)).astype(np.float32)


def _sigmoid_of_normal(rng, shape):
    z = rng.standard_normal(size=shape, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def make_inputs(cell: str, B: int, T: int, D: int, dtype: str = "f32", seed: int = 0,
                with_grad: bool = False, head_size: int | None = None) -> Inputs:
    """Draw one problem of the given shape with the benchmark distributions.

    Draw order: pre-activation planes in gate order, then recurrent weights
    [G][D] (head_gru: [3][D/hs][hs][hs]), then biases [G][D], then (if asked) the
    upstream gradient.
    Gate orders: gru (z, r, c); lstm (i, f, o, g); slstm (z, i, f, o); linear (a, b).
    Biases ~ N(0, 0.1^2), except the forget gate's (lstm, slstm), which is 1.
    """
    assert cell in GATES and dtype in ("f32", "bf16")
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, T, D)
    G = GATES[cell]
    w = bias = None
    if cell == "linear":
        a = _sigmoid_of_normal(rng, shape)
        b = _normal(rng, shape)
        pre = [a, b]
    else:
        pre = [_normal(rng, shape) for _ in range(G)]
        if cell == "head_gru":
            assert head_size is not None and head_size >= 1 and D % head_size == 0
            w = (_uniform_half(rng, (G, D // head_size, head_size, head_size)) *
                 np.float32(2.0 / np.sqrt(head_size))).astype(np.float32)
        else:
            w = _uniform_half(rng, (G, D))
        if cell in ("gru", "head_gru"):
            bias = (rng.standard_normal(size=(G, D), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
        elif cell == "slstm":
            drawn = (rng.standard_normal(size=(3, D), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
            bias = np.empty((4, D), dtype=np.float32)
            bias[0], bias[1], bias[3] = drawn[0], drawn[1], drawn[2]   # z, i, o
            bias[2] = 1.0                                               # forget gate
        else:
            drawn = (rng.standard_normal(size=(3, D), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
            bias = np.empty((4, D), dtype=np.float32)
            bias[0], bias[2], bias[3] = drawn[0], drawn[1], drawn[2]   # i, o, g
            bias[1] = 1.0                                               # forget gate
    if dtype == "bf16":
        pre = [f32_to_bf16_bits(p) for p in pre]
    g = _normal(rng, shape) if with_grad else None
    return Inputs(cell, B, T, D, dtype, pre, w, bias, g, head_size if cell == "head_gru" else 1)


def workload_inputs(wl: Workload, seed: int | None = None, B=None, T=None, D=None) -> Inputs:
    """Inputs for a benchmark workload (seed defaults to its index); shape may be overridden."""
    return make_inputs(wl.cell, B or wl.B, T or wl.T, D or wl.D, wl.dtype,
                       wl.index if seed is None else seed, with_grad=wl.vjp)


def random_state(S: int, B: int, D: int, seed: int, scale: float = 0.5) -> np.ndarray:
    """A random initial state s0 [S][B][D] (for tests of nonzero initial states)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(size=(S, B, D), dtype=np.float32) * np.float32(scale)).astype(np.float32)


def packed_offsets(T: int, seed: int, mean_len: float, forced=()) -> np.ndarray:
    """Offsets cu_seqlens (int32, first 0, last T) of sequences packed along T: lengths drawn from a
    geometric distribution with the given mean (so short and long sequences mix, as in packed
    training batches), plus the boundaries listed in `forced`.  Empty sequences are kept when two
    offsets coincide."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cuts = [0]
    while cuts[-1] < T:
        cuts.append(cuts[-1] + int(rng.geometric(1.0 / max(mean_len, 1.0))))
    cuts[-1] = T
    cuts = sorted(cuts + [int(f) for f in forced if 0 <= int(f) <= T])
    return np.asarray(cuts, dtype=np.int32)
