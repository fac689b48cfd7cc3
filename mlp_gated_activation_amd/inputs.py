"""Seeded synthetic inputs for the gated activation (no activation math here).

Every tensor is drawn in float32 on the CPU from one ``torch.Generator``
seeded per workload, in the order each function lists, and then rounded
(round-to-nearest-even, by ``Tensor.to``) to the storage dtype.  The same
rounded tensors feed both the GPU library and the fp64 oracle, so nothing
here depends on either.

Shapes follow the workloads the pages describe:

* "Write a Triton SiLU-Mul (SwiGLU) Kernel", "Inputs the agent should gather
  first", items 3, 4 and 9: ``(B*T, I)`` activations with I = 11008, 14336 or
  18944, split or fused ``[gate | up]``.
* "Kernel Profile: SwiGLU (Tier 1 -- Element-wise)", "Benchmarking": bf16,
  B*T = 4096, hidden size swept over 1024 ... 16384.

These are synthetic stand-ins for model activations; no dataset or weights
are involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(seed)


def separate(rows: int, cols: int, dtype: str, a_std: float = 2.0, seed: int = 0):
    """Separate a, b, dy of shape (rows, cols).

    Draw order: ``a = a_std*randn``, ``b = randn``, ``dy = randn``.
    """
    g = _gen(seed)
    t = DTYPES[dtype]
    a = (torch.randn(rows, cols, generator=g) * a_std).to(t)
    b = torch.randn(rows, cols, generator=g).to(t)
    dy = torch.randn(rows, cols, generator=g).to(t)
    return a, b, dy


def gate_up(rows: int, cols: int, dtype: str, x_std: float = 1.5, seed: int = 0):
    """Fused x = [a | b] of shape (rows, 2*cols) and dy of shape (rows, cols).

    Draw order: ``x = x_std*randn(rows, 2*cols)``, ``dy = randn(rows, cols)``.
    """
    g = _gen(seed)
    t = DTYPES[dtype]
    x = (torch.randn(rows, 2 * cols, generator=g) * x_std).to(t)
    dy = torch.randn(rows, cols, generator=g).to(t)
    return x, dy


def gate_up_stress(rows: int, cols: int, dtype: str, frac: float = 0.01,
                   lo: float = 20.0, hi: float = 80.0, seed: int = 0):
    """Fused x = [a | b] whose gate half mixes N(0,1) with rare large values.

    Per element of a: with probability ``frac`` a magnitude uniform in
    [lo, hi] with a random sign, else N(0, 1).  Draw order: ``g = randn``,
    ``m = rand < frac``, ``mag = lo + (hi-lo)*rand``, ``sgn = rand < 0.5``
    (-1 where true), ``b = randn``, ``dy = randn``; all (rows, cols).
    """
    gen = _gen(seed)
    t = DTYPES[dtype]
    g = torch.randn(rows, cols, generator=gen)
    m = torch.rand(rows, cols, generator=gen) < frac
    mag = lo + (hi - lo) * torch.rand(rows, cols, generator=gen)
    sgn = torch.where(torch.rand(rows, cols, generator=gen) < 0.5, -1.0, 1.0)
    a = torch.where(m, sgn * mag, g)
    del g, mag, sgn
    b = torch.randn(rows, cols, generator=gen)
    x = torch.cat([a, b], dim=1).to(t)
    del a, b
    dy = torch.randn(rows, cols, generator=gen).to(t)
    return x, dy


def add_rmsnorm(rows: int, hidden: int, dtype: str, seed: int = 0):
    """x, residual of shape (rows, hidden) and gamma (hidden,) for the fused
    residual add + RMSNorm ("Write a Triton Fused Add+RMSNorm Kernel").

    Draw order: ``x = randn``, ``residual = randn``, ``gamma = 1 + 0.1*randn``.
    """
    g = _gen(seed)
    t = DTYPES[dtype]
    x = torch.randn(rows, hidden, generator=g).to(t)
    res = torch.randn(rows, hidden, generator=g).to(t)
    gamma = (1.0 + 0.1 * torch.randn(hidden, generator=g)).to(t)
    return x, res, gamma


def gemm_glu(M: int, N: int, K: int, dtype: str, w_std: float = 0.02, seed: int = 0):
    """x (M, K) and a fused [gate | up] weight w (2N, K) for the gate/up
    projection with the fused activation ("Fused Kernels", section 4).
    Draw order: ``x = randn(M, K)``, ``w = w_std * randn(2N, K)`` (the usual
    0.02 initialisation of a linear layer, so g and u are about N(0, K*w_std^2)).
    """
    g = _gen(seed)
    t = DTYPES[dtype]
    x = torch.randn(M, K, generator=g).to(t)
    w = (torch.randn(2 * N, K, generator=g) * w_std).to(t)
    return x, w


def gemm_glu_exact(M: int, N: int, K: int, dtype: str, seed: int = 0):
    """Inputs of the gate/up projection whose sums are exact in fp32 in any
    order: x (M, K) of integers uniform in [-8, 8] and w (2N, K) of integers
    uniform in [-8, 8] times 2^-8.  Every product is a multiple of 2^-8 of
    magnitude at most 1/4, so every partial sum over K <= 2^16 terms is a
    multiple of 2^-8 below 2^14 in magnitude, which fp32 holds exactly.
    Draw order: ``x = randint(-8, 9, (M, K))``, ``w = randint(-8, 9, (2N, K))``."""
    if K > (1 << 16):
        raise ValueError("K above 2^16: partial sums could leave fp32's exact range")
    g = _gen(seed)
    t = DTYPES[dtype]
    x = torch.randint(-8, 9, (M, K), generator=g).to(t)
    w = (torch.randint(-8, 9, (2 * N, K), generator=g).to(torch.float32) * 2.0 ** -8).to(t)
    return x, w


def all_bit_patterns(dtype: str) -> torch.Tensor:
    """Every 16-bit pattern of a 16-bit dtype, in bit order, as a 1-D tensor."""
    t = DTYPES[dtype]
    if t.itemsize != 2:
        raise ValueError("only 16-bit dtypes")
    return torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(t)


@dataclass(frozen=True)
class Workload:
    """One named workload: kind(s), dtype, layout and shape."""
    name: str
    kinds: tuple
    dtype: str
    layout: str            # "separate" or "gate_up"
    rows: int
    cols: int              # activation width I (the b half of x in gate_up)
    std: float = 2.0       # std of a (separate) or x (gate_up)
    stress: bool = False   # gate half mixes in rare large values
    notes: str = field(default="", compare=False)

    def make(self, seed: int = 0):
        """Returns ``(a, b, dy)`` for separate, ``(x, dy)`` for gate_up."""
        if self.layout == "separate":
            return separate(self.rows, self.cols, self.dtype, self.std, seed)
        if self.stress:
            return gate_up_stress(self.rows, self.cols, self.dtype, seed=seed)
        return gate_up(self.rows, self.cols, self.dtype, self.std, seed)

    @property
    def elements(self) -> int:
        return self.rows * self.cols


WORKLOADS = {
    w.name: w for w in [
        Workload("swiglu_f32_64x1024", ("silu",), "fp32", "separate", 64, 1024, 2.0,
                 notes="tiny fp32 case; finite-difference backward check"),
        Workload("swiglu_bf16_4096x11008", ("silu",), "bf16", "separate", 4096, 11008, 2.0,
                 notes="LLaMA-7B-like intermediate width"),
        Workload("swiglu_bf16_gateup_4096x14336", ("silu",), "bf16", "gate_up", 4096, 14336, 1.5,
                 notes="fused [gate|up] x of shape (4096, 28672)"),
        *[Workload(f"swiglu_bf16_4096x{h}", ("silu",), "bf16", "separate", 4096, h, 2.0,
                   notes="hidden-size sweep") for h in (1024, 2048, 4096, 8192, 16384)],
        Workload("swiglu_bf16_tp8_4096x1792", ("silu",), "bf16", "separate", 4096, 1792, 2.0,
                 notes="one tensor-parallel rank's share of I = 14336 at TP = 8"),
        Workload("geglu_reglu_fp16_gateup_8191x18944", ("gelu_erf", "gelu_tanh", "relu"), "fp16",
                 "gate_up", 8191, 18944, 1.0, stress=True,
                 notes="odd row count, Qwen2-7B-like width, 1% large gate values"),
        Workload("swiglu_bf16_4096x14336", ("silu",), "bf16", "separate", 4096, 14336, 2.0,
                 notes="headline: fwd out-of-place then bwd in place"),
    ]
}
