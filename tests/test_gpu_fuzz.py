"""Seeded random cases for the row-major entry points, the gate/up GEMM and
the add + RMSNorm forward, through the binding and the C ABI, against the
fp64 oracle at the bounds of their own parity tests.

Row-major glu_fwd / glu_bwd: a shape (rows 1..300, cols 1..600,
log-uniform), dtype, kind, layout (separate or [gate | up]), direction, in
place or not, and for every operand a padded row stride and a base offset
that decides between the 16-byte vector path and the element path.  Operands
live inside sentinel-filled buffers: everything outside the written views
must keep its sentinels ("Write a Triton SiLU-Mul (SwiGLU) Kernel", Kernel
design rules: always mask; Common failure modes: in-place stores).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import compare
from gemm_bounds import pre_bound
from test_gpu_gemm import check_h
from test_gpu_rmsnorm import check_all

pytestmark = pytest.mark.gpu

KINDS = ("silu", "gelu_erf", "gelu_tanh", "relu")
DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
SENTINEL = 12288.0   # exact in every dtype here


@pytest.fixture(scope="module")
def glu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conftest import ensure_built
    ensure_built()
    from mlp_gated_activation_amd import glu as g
    return g


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def logu(rng, hi):
    return int(round(np.exp(rng.uniform(0, np.log(hi)))))


class Canvas:
    """A (rows, width) view with row stride ld at element offset off inside a
    sentinel-filled device buffer."""

    def __init__(self, rows, width, ld, off, dtype, values=None):
        n = off + (rows - 1) * ld + width + 13
        buf = torch.full((n,), SENTINEL, dtype=dtype)
        view = buf.as_strided((rows, width), (ld, 1), off)
        if values is not None:
            view.copy_(values)
        self.buf = buf.cuda()
        self.view = self.buf.as_strided((rows, width), (ld, 1), off)
        mask = torch.zeros(n, dtype=torch.bool)
        idx = torch.arange(n).as_strided((rows, width), (ld, 1), off)
        mask[idx.reshape(-1)] = True
        self.mask = mask

    def outside_untouched(self, what):
        rest = self.buf.cpu()[~self.mask].to(torch.float64)
        assert bool((rest == SENTINEL).all()), f"{what}: wrote outside the view"


def check(got, ref, fmt, what, exact):
    g = f64(got)
    rep = compare(g, ref, fmt)
    assert rep.ok, f"{what}: {rep}"
    if exact:
        want = torch.from_numpy(np.ascontiguousarray(ref)).to(torch.float32).to(got.dtype).to(torch.float64)
        gg = torch.from_numpy(g)
        assert bool(((gg == want) | (torch.isnan(gg) & torch.isnan(want))).all()), f"{what}: not RNE(exact)"


def rowmajor_case(seed):
    rng = np.random.default_rng(2000 + seed)
    R, C = logu(rng, 300), logu(rng, 600)
    dtype = ("bf16", "fp16", "fp32")[rng.integers(3)]
    return dict(R=R, C=C, dtype=dtype, kind=KINDS[rng.integers(4)], gate_up=bool(rng.integers(2)),
                bwd=bool(rng.integers(2)), inplace=bool(rng.integers(2)),
                pads=[int(rng.integers(0, 18)) for _ in range(5)], offs=[int(rng.integers(0, 8)) for _ in range(5)])


@pytest.mark.parametrize("seed", range(120))
def test_random_rowmajor(glu, seed):
    p = rowmajor_case(seed)
    R, C, dt, kind = p["R"], p["C"], DT[p["dtype"]], p["kind"]
    what = f"seed {seed}: {p}"
    print(what, flush=True)
    g = torch.Generator().manual_seed(seed)
    a = (torch.randn(R, C, generator=g) * 2).to(dt)
    b = torch.randn(R, C, generator=g).to(dt)
    dy = torch.randn(R, C, generator=g).to(dt)
    fa, fb, fdy = f64(a), f64(b), f64(dy)
    pads, offs = p["pads"], p["offs"]
    exact = kind == "relu"
    if p["gate_up"]:
        X = Canvas(R, 2 * C, 2 * C + pads[0], offs[0], dt, torch.cat([a, b], 1))
        xa, xb = X.view[:, :C], X.view[:, C:]
    else:
        A = Canvas(R, C, C + pads[0], offs[0], dt, a)
        B = Canvas(R, C, C + pads[1], offs[1], dt, b)
    lay = "gate_up" if p["gate_up"] else "separate"
    if not p["bwd"]:
        ref = oracle.fwd(kind, fa, fb)
        if p["inplace"]:
            out = glu.glu_fwd(kind, lay, X.view if p["gate_up"] else A.view, None if p["gate_up"] else B.view,
                              inplace=True)
            check(out, ref, p["dtype"], what + " y in place", exact)
            (X if p["gate_up"] else B).outside_untouched(what)
            if p["gate_up"]:
                check(xa, fa, p["dtype"], what + " gate kept", True)
        else:
            Y = Canvas(R, C, C + pads[2], offs[2], dt)
            glu.glu_fwd(kind, lay, X.view if p["gate_up"] else A.view, None if p["gate_up"] else B.view, y=Y.view)
            check(Y.view, ref, p["dtype"], what + " y", exact)
            Y.outside_untouched(what + " y")
    else:
        D = Canvas(R, C, C + pads[3], offs[3], dt, dy)
        rda, rdb = oracle.bwd(kind, fa, fb, fdy)
        if p["gate_up"]:
            if p["inplace"]:
                glu.glu_bwd(kind, lay, X.view, None, D.view, inplace=True)
                outa, outb, canv = xa, xb, [X]
            else:
                DX = Canvas(R, 2 * C, 2 * C + pads[4], offs[4], dt)
                glu.glu_bwd(kind, lay, X.view, None, D.view, da=DX.view, inplace=False)
                outa, outb, canv = DX.view[:, :C], DX.view[:, C:], [DX]
        else:
            if p["inplace"]:
                glu.glu_bwd(kind, lay, A.view, B.view, D.view, inplace=True)
                outa, outb, canv = A.view, B.view, [A, B]
            else:
                DA = Canvas(R, C, C + pads[2], offs[2], dt)
                DB = Canvas(R, C, C + pads[4], offs[4], dt)
                glu.glu_bwd(kind, lay, A.view, B.view, D.view, da=DA.view, db=DB.view, inplace=False)
                outa, outb, canv = DA.view, DB.view, [DA, DB]
        check(outa, rda, p["dtype"], what + " da", exact)
        check(outb, rdb, p["dtype"], what + " db", exact)
        for c in canv:
            c.outside_untouched(what)
        D.outside_untouched(what + " dy")


def gemm_case(seed):
    rng = np.random.default_rng(3000 + seed)
    return dict(M=logu(rng, 700), N=logu(rng, 700), K=8 * logu(rng, 140), dtype=("bf16", "fp16")[rng.integers(2)],
                kind=KINDS[rng.integers(4)], gu=bool(rng.integers(2)), padx=8 * int(rng.integers(0, 4)),
                padw=8 * int(rng.integers(0, 4)))


@pytest.mark.parametrize("seed", range(40))
def test_random_gemm(glu, seed):
    p = gemm_case(seed)
    M, N, K, dt = p["M"], p["N"], p["K"], DT[p["dtype"]]
    what = f"seed {seed}: {p}"
    print(what, flush=True)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(dt)
    w = (torch.randn(2 * N, K, generator=g) * 0.1).to(dt)
    xb = torch.zeros(M, K + p["padx"], dtype=dt)
    xb[:, :K] = x
    wb = torch.zeros(2 * N, K + p["padw"], dtype=dt)
    wb[:, :K] = w
    gx, gw = xb.cuda()[:, :K], wb.cuda()[:, :K]
    if p["gu"]:
        h, gu = glu.glu_gemm_fwd(p["kind"], gx, gw, gu=True)
    else:
        h = glu.glu_gemm_fwd(p["kind"], gx, gw)
    torch.cuda.synchronize()
    # the edge-shape bar of the GEMM parity tests: tiny K leaves more results a hair past one ulp
    check_h(h, x, w[:N], w[N:], p["kind"], what, min_one_ulp=0.95)
    if p["gu"]:
        _, gref, uref = oracle.gemm_glu(p["kind"], f64(x), f64(w[:N]), f64(w[N:]), want_gu=True)
        for name, got, want, wt in (("g", gu[:, :N], gref, w[:N]), ("u", gu[:, N:], uref, w[N:])):
            err = np.abs(f64(got) - want)
            assert (err <= pre_bound(p["dtype"], K, f64(x), f64(wt), want)).all(), f"{what} {name}"


def rms_case(seed):
    rng = np.random.default_rng(4000 + seed)
    return dict(rows=logu(rng, 200), H=logu(rng, 20000), dtype=("bf16", "fp16", "fp32")[rng.integers(3)],
                pad=int(rng.integers(0, 9)), eps=(1e-6, 1e-5)[rng.integers(2)], rstd=bool(rng.integers(2)))


@pytest.mark.parametrize("seed", range(40))
def test_random_rmsnorm(glu, seed):
    p = rms_case(seed)
    R, H, dt = p["rows"], p["H"], DT[p["dtype"]]
    what = f"seed {seed}: {p}"
    print(what, flush=True)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(R, H, generator=g).to(dt)
    r = torch.randn(R, H, generator=g).to(dt)
    gamma = (1 + 0.1 * torch.randn(H, generator=g)).to(dt)
    X = Canvas(R, H, H + p["pad"], 0, dt, x)
    RR = Canvas(R, H, H + p["pad"], 0, dt, r)
    h, y, rstd = glu.glu_add_rmsnorm_fwd(X.view, RR.view, gamma.cuda(), p["eps"], rstd=p["rstd"])
    torch.cuda.synchronize()
    check_all(h, y, rstd, x, r, gamma, p["eps"], what)
    X.outside_untouched(what + " x")
    RR.outside_untouched(what + " residual")
