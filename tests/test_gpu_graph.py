"""HIP graph capture of the strided, GEMM and add + RMSNorm entry points.

None of them allocates or issues a memset, so their launches capture into a
graph.  The graph is replayed several times with new inputs and eager work
(and synchronisations) between the replays; every replay must equal the
eager launches bit for bit, and the eager results are checked against the
fp64 oracle once, so that the comparison is not between two wrong results.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import compare

pytestmark = pytest.mark.gpu

FMT = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}


@pytest.fixture(scope="module")
def glu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conftest import ensure_built
    ensure_built()
    from mlp_gated_activation_amd import glu as g
    return g


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def same_bits(got: torch.Tensor, want: torch.Tensor) -> bool:
    if got.dtype == torch.float32:
        return torch.equal(got.view(torch.int32), want.view(torch.int32))
    return torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_graph_replay_strided_gemm_rmsnorm(glu):
    t = torch.bfloat16
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(41)
    # strided: R x C views with ragged tiles; dy and one output transposed
    R, C = 520, 1000
    a = torch.empty(R, C, dtype=t, device=dev)
    b = torch.empty_like(a)
    dyT = torch.empty(C, R, dtype=t, device=dev)
    dy = dyT.t()
    yT = torch.empty(C, R, dtype=t, device=dev)
    y = yT.t()
    da = torch.empty_like(a)
    db = torch.empty_like(a)
    # GEMM: ragged in every dimension, with the [gate | up] pre-activations
    M, N, K = 300, 200, 136
    x = torch.empty(M, K, dtype=t, device=dev)
    w = torch.empty(2 * N, K, dtype=t, device=dev)
    h = torch.empty(M, N, dtype=t, device=dev)
    gu = torch.empty(M, 2 * N, dtype=t, device=dev)
    # add + RMSNorm: rows of a width that is not a multiple of the vector
    RR, H = 257, 3000
    xr = torch.empty(RR, H, dtype=t, device=dev)
    res = torch.empty_like(xr)
    gamma = torch.empty(H, dtype=t, device=dev)
    hr = torch.empty_like(xr)
    yr = torch.empty_like(xr)
    rstd = torch.empty(RR, dtype=torch.float32, device=dev)
    # the few-token GEMM tiles (M <= 256) and the multi-row add + RMSNorm
    # kernel (8192-wide rows, 37 rows over 10 workgroups)
    Ms = 100
    hs = torch.empty(Ms, N, dtype=t, device=dev)
    RW, HW = 37, 8192
    xw = torch.empty(RW, HW, dtype=t, device=dev)
    rw = torch.empty_like(xw)
    gw = torch.empty(HW, dtype=t, device=dev)
    hw = torch.empty_like(xw)
    yw = torch.empty_like(xw)

    def refill():
        a.copy_(torch.randn(R, C, device=dev, generator=g) * 2)
        b.copy_(torch.randn(R, C, device=dev, generator=g))
        dyT.copy_(torch.randn(C, R, device=dev, generator=g))
        x.copy_(torch.randn(M, K, device=dev, generator=g))
        w.copy_(torch.randn(2 * N, K, device=dev, generator=g) * 0.1)
        xr.copy_(torch.randn(RR, H, device=dev, generator=g))
        res.copy_(torch.randn(RR, H, device=dev, generator=g))
        gamma.copy_(1 + 0.1 * torch.randn(H, device=dev, generator=g))
        xw.copy_(torch.randn(RW, HW, device=dev, generator=g))
        rw.copy_(torch.randn(RW, HW, device=dev, generator=g))
        gw.copy_(1 + 0.1 * torch.randn(HW, device=dev, generator=g))

    def launch(out_y, out_da, out_db, out_h, out_gu, out_hr, out_yr, out_rstd, out_hs, out_hw, out_yw):
        glu.glu_fwd_strided("silu", a, b, out_y)
        glu.glu_bwd_strided("gelu_erf", a, b, dy, out_da, out_db)
        glu.glu_gemm_fwd("silu", x, w, h=out_h, gu=out_gu)
        glu.glu_add_rmsnorm_fwd(xr, res, gamma, 1e-6, h=out_hr, y=out_yr, rstd=out_rstd)
        glu.glu_gemm_fwd("gelu_tanh", x[:Ms], w, h=out_hs)
        glu.glu_add_rmsnorm_fwd(xw, rw, gw, 1e-6, h=out_hw, y=out_yw)

    outs = (y, da, db, h, gu, hr, yr, rstd, hs, hw, yw)
    refill()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch(*outs)
    eager = [torch.empty_like(v) for v in outs]
    for rep in range(4):
        refill()
        graph.replay()
        torch.cuda.synchronize()
        launch(*eager)
        torch.cuda.synchronize()
        for got, want, nm in zip(outs, eager, ("y", "da", "db", "h", "gu", "h (norm)", "y (norm)", "rstd",
                                               "h (few tokens)", "h (8192-wide norm)", "y (8192-wide norm)")):
            assert same_bits(got, want), f"replay {rep}: {nm} differs from the eager launch"

    # the eager results of the last round against the oracle
    fa, fb, fdy = f64(a), f64(b), f64(dy)
    for got, ref, nm in ((y, oracle.fwd("silu", fa, fb), "strided fwd"),):
        rep = compare(f64(got), ref, FMT[got.dtype])
        assert rep.ok, f"{nm}: {rep}"
    rda, rdb = oracle.bwd("gelu_erf", fa, fb, fdy)
    for got, ref, nm in ((da, rda, "strided da"), (db, rdb, "strided db")):
        rep = compare(f64(got), ref, FMT[got.dtype])
        assert rep.ok, f"{nm}: {rep}"
    rh, _, _ = oracle.gemm_glu("silu", f64(x), f64(w[:N]), f64(w[N:]), want_gu=True)
    # the GEMM bound is checked in its own tests; here the accumulation at
    # K = 136 keeps every result within a few output ulps of the oracle
    err = np.abs(f64(h) - rh)
    assert float(np.max(err / np.maximum(np.abs(rh), 1e-3))) < 2 ** -6, "GEMM h far from the oracle"
    ref = oracle.add_rmsnorm(f64(xr), f64(res), f64(gamma), 1e-6)
    rep = compare(f64(yr), ref[1], FMT[yr.dtype])
    assert rep.ok, f"add_rmsnorm y: {rep}"
    ref = oracle.add_rmsnorm(f64(xw), f64(rw), f64(gw), 1e-6)
    for got, want, nm in ((hw, ref[0], "h"), (yw, ref[1], "y")):
        rep = compare(f64(got), want, FMT[got.dtype])
        assert rep.ok, f"8192-wide add_rmsnorm {nm}: {rep}"
    rhs, _, _ = oracle.gemm_glu("gelu_tanh", f64(x[:Ms]), f64(w[:N]), f64(w[N:]), want_gu=True)
    err = np.abs(f64(hs) - rhs)
    assert float(np.max(err / np.maximum(np.abs(rhs), 1e-3))) < 2 ** -6, "few-token GEMM h far from the oracle"
