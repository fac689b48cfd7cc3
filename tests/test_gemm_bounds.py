"""CPU checks of the gate/up GEMM's error bound (gemm_bounds.py) against
an independent, plainly faithful emulation of the contract it is derived
from: fp32 accumulation of the exact products in a fixed order (forward
and reversed), the activation and the product in fp32 (torch's float32
CPU functions), one round-to-nearest to the 16-bit type.  The emulation
must sit inside the bound everywhere, and a result moved by two output
ulps must fall outside it wherever the accumulation term is small (short
sums), so the bound is neither violated by a faithful implementation nor
vacuous.  (For long sums the worst-case accumulation term dominates; the
GPU tests add a strict one-ulp check on inputs whose sums are exact.)"""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from gemm_bounds import h_bound, pre_bound
from oracle.compare import FORMATS, ulp

DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
ACT32 = {"silu": F.silu, "gelu_erf": lambda t: F.gelu(t), "gelu_tanh": lambda t: F.gelu(t, approximate="tanh"),
         "relu": F.relu}


def emulate(kind, x, wg, wu, dtype, reverse):
    """h, g, u as a faithful fp32-accumulating kernel computes them."""
    x32, g32w, u32w = (t.to(torch.float32).numpy() for t in (x, wg, wu))
    K = x32.shape[1]
    g = np.zeros((x32.shape[0], g32w.shape[0]), np.float32)
    u = np.zeros_like(g)
    for k in (range(K - 1, -1, -1) if reverse else range(K)):
        g += np.outer(x32[:, k], g32w[:, k])   # products of 16-bit values: exact in fp32
        u += np.outer(x32[:, k], u32w[:, k])
    gt, ut = torch.from_numpy(g), torch.from_numpy(u)
    h = (ACT32[kind](gt) * ut).to(DT[dtype])
    return h.to(torch.float64).numpy(), gt.to(DT[dtype]).to(torch.float64).numpy(), \
        ut.to(DT[dtype]).to(torch.float64).numpy()


@pytest.mark.parametrize("K", [16, 1024])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("kind", ["silu", "gelu_erf", "gelu_tanh", "relu"])
def test_faithful_emulation_within_bound(kind, dtype, K):
    gen = torch.Generator().manual_seed(21)
    M, N = 48, 40
    x = torch.randn(M, K, generator=gen).to(DT[dtype])
    w = (0.05 * torch.randn(2 * N, K, generator=gen)).to(DT[dtype])
    # two rows whose gate sums cancel: x row 1 = -x row 0 on the second half of k
    x[1, : K // 2] = x[0, : K // 2]
    x[1, K // 2:] = -x[0, K // 2:]
    wg, wu = w[:N], w[N:]
    fx, fg, fu = (t.to(torch.float64).numpy() for t in (x, wg, wu))
    ref, g, u = oracle.gemm_glu(kind, fx, fg, fu, want_gu=True)
    bound = h_bound(dtype, K, fx, fg, fu, ref, g, u, oracle.act(kind, g))
    for reverse in (False, True):
        h, gq, uq = emulate(kind, x, wg, wu, dtype, reverse)
        assert (np.abs(h - ref) <= bound).all(), (kind, dtype, reverse)
        assert (np.abs(gq - g) <= pre_bound(dtype, K, fx, fg, g)).all()
        assert (np.abs(uq - u) <= pre_bound(dtype, K, fx, fu, u)).all()
    # not vacuous: where the accumulation term is small (short sums), two
    # output ulps off fall outside it
    step = ulp(ref, FORMATS[dtype])
    tight = bound - step < 0.5 * step
    if K == 16:
        assert tight[ref != 0].mean() > 0.9   # (ReLU's exact zeros sit at the subnormal floor)
    assert (np.abs(h + 2 * step - ref) > bound)[tight].all()
