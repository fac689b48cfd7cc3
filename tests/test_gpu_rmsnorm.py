"""GPU parity of the fused residual add + RMSNorm forward against the fp64
oracle ("Write a Triton Fused Add+RMSNorm Kernel").

h and y: within one output ulp of the exact values (h = x + residual,
y = h * rstd * gamma).  rstd (fp32): relative error at most 8e-6 for
bf16/fp16 data (fp32 accumulation: at most ~86 sequential roundings in the
sum of squares, halved by the square root, plus 3 roundings) and 1e-6 for
fp32 data (fp64 accumulation)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import compare
from mlp_gated_activation_amd import inputs

pytestmark = pytest.mark.gpu
FMT = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}
DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


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


def check_all(h, y, rstd, x, r, g, eps, what):
    fmt = FMT[x.dtype]
    eps32 = float(np.float32(eps))
    rh, ry, rr = oracle.add_rmsnorm(f64(x), f64(r), f64(g), eps32)
    for got, ref, nm in ((h, rh, "h"), (y, ry, "y")):
        rep = compare(f64(got), ref, fmt)
        assert rep.ok, f"{what} {nm}: {rep}"
    if rstd is not None:
        tol = 1e-6 if x.dtype == torch.float32 else 8e-6
        rel = np.abs(f64(rstd).reshape(-1) - rr) / rr
        assert rel.max() <= tol, f"{what} rstd: max rel {rel.max():.3g} at row {int(rel.argmax())}"


@pytest.mark.parametrize("hidden", [4096, 8192])
def test_workload_bf16(glu, hidden):
    x, r, g = inputs.add_rmsnorm(4096, hidden, "bf16")
    gx, gr, gg = x.cuda(), r.cuda(), g.cuda()
    h, y, rstd = glu.glu_add_rmsnorm_fwd(gx, gr, gg, 1e-6, rstd=True)
    check_all(h, y, rstd, x, r, g, 1e-6, f"bf16 4096x{hidden}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rows,hidden", [(5120, 4096), (6144, 4096), (8192, 3000), (16384, 4096)])
def test_gamma_early_and_late(glu, dtype, rows, hidden):
    """The 64-thread, 8-vector shape with gamma loaded late (5120 rows, where
    the early-gamma instance would need a second round of rows on 256 CUs)
    and early (6144 rows; 8192 x 3000, rows shorter than the shape's 4096)."""
    x, r, g = inputs.add_rmsnorm(rows, hidden, dtype, seed=3)
    gx, gr, gg = x.cuda(), r.cuda(), g.cuda()
    h, y, rstd = glu.glu_add_rmsnorm_fwd(gx, gr, gg, 1e-6, rstd=True)
    check_all(h, y, rstd, x, r, g, 1e-6, f"{dtype} {rows}x{hidden}")


HIDDEN = [1, 7, 8, 100, 512, 513, 1024, 2048, 2049, 4096, 5120, 8192, 16384, 16385, 32768, 65536, 65544, 70000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_every_kernel_shape(glu, dtype):
    """Widths that land on each block/vector shape and on the two-pass kernel,
    aligned (vector path) and one element off (element path)."""
    t = DT[dtype]
    for hidden in HIDDEN:
        rows = 3 if hidden > 8192 else 17
        x, r, g = inputs.add_rmsnorm(rows, hidden, dtype, seed=hidden)
        for off in (0, 1):
            bx = torch.zeros(rows * hidden + 8, dtype=t, device="cuda")
            br = torch.zeros_like(bx)
            bg = torch.zeros(hidden + 8, dtype=t, device="cuda")
            gx = bx[off:off + rows * hidden].view(rows, hidden)
            gr = br[off:off + rows * hidden].view(rows, hidden)
            gg = bg[off:off + hidden]
            gx.copy_(x.cuda()); gr.copy_(r.cuda()); gg.copy_(g.cuda())
            h, y, rstd = glu.glu_add_rmsnorm_fwd(gx, gr, gg, 1e-5, rstd=True)
            check_all(h, y, rstd, x, r, g, 1e-5, f"{dtype} {rows}x{hidden} off={off}")


SENT = {torch.bfloat16: 0x7FA5, torch.float16: 0x7DA5, torch.float32: 0x7FA5A5A5}


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_strided_rows_inplace_and_canaries(glu, dtype):
    """Row strides wider than hidden, h written over x (in-place residual
    update) or over residual, y over x, with sentinels around every output."""
    t = DT[dtype]
    ib = torch.int32 if t == torch.float32 else torch.int16
    for hidden, rows in ((1000, 9), (4096, 5), (8192, 6), (70000, 2)):
        x, r, g = inputs.add_rmsnorm(rows, hidden, dtype, seed=7)
        ld = hidden + 24
        for mode in ("separate", "h_over_x", "h_over_res", "y_over_x"):
            if hidden > 65536 // (2 if t == torch.float32 else 1) and mode in ("h_over_x", "h_over_res"):
                continue   # the two-pass kernel needs x and residual intact (tested in test_two_pass_rejects)
            bufs = {n: torch.full(((rows + 2) * ld,), SENT[t], dtype=ib, device="cuda").view(t)
                    for n in ("x", "r", "h", "y")}
            view = {n: b[ld:ld + rows * ld].view(rows, ld)[:, :hidden] for n, b in bufs.items()}
            view["x"].copy_(x.cuda()); view["r"].copy_(r.cuda())
            gg = g.cuda()
            rbuf = torch.full((rows + 8,), float("nan"), dtype=torch.float32, device="cuda")
            hv = {"h_over_x": view["x"], "h_over_res": view["r"]}.get(mode, view["h"])
            yv = view["x"] if mode == "y_over_x" else view["y"]
            glu.glu_add_rmsnorm_fwd(view["x"], view["r"], gg, 1e-6, h=hv, y=yv, rstd=rbuf[4:4 + rows])
            check_all(hv, yv, rbuf[4:4 + rows], x, r, g, 1e-6, f"{dtype} {rows}x{hidden} {mode}")
            assert torch.isnan(rbuf[:4]).all() and torch.isnan(rbuf[4 + rows:]).all(), "rstd canary"
            for n, b in bufs.items():
                mask = torch.ones(b.numel(), dtype=torch.bool)
                idx = (ld + torch.arange(rows)[:, None] * ld + torch.arange(hidden)[None, :]).reshape(-1)
                mask[idx] = False
                bits = b.view(ib).cpu()[mask]
                assert bool((bits == SENT[t]).all()), f"{dtype} {mode}: buffer {n} written outside its rows"


def test_eps_and_zero_rows(glu):
    x, r, g = inputs.add_rmsnorm(6, 2048, "bf16", seed=11)
    x[2] = 0
    r[2] = 0
    for eps in (1e-6, 1e-2, 0.5):
        h, y, rstd = glu.glu_add_rmsnorm_fwd(x.cuda(), r.cuda(), g.cuda(), eps, rstd=True)
        check_all(h, y, rstd, x, r, g, eps, f"eps={eps}")
        assert bool((y[2] == 0).all())


def test_two_pass_rejects_h_over_x(glu):
    x, r, g = inputs.add_rmsnorm(2, 70000, "bf16", seed=13)
    gx, gr = x.cuda(), r.cuda()
    with pytest.raises(glu.GluError, match="GLU_ERR_ALIAS"):
        glu.glu_add_rmsnorm_fwd(gx, gr, g.cuda(), 1e-6, h=gx)
    with pytest.raises(glu.GluError, match="GLU_ERR_ARG"):
        glu.glu_add_rmsnorm_fwd(gx, gr, g.cuda(), 0.0)


def test_3d_input_and_no_rstd(glu):
    x, r, g = inputs.add_rmsnorm(4 * 37, 1536, "fp16", seed=17)
    h, y, rstd = glu.glu_add_rmsnorm_fwd(x.view(4, 37, 1536).cuda(), r.view(4, 37, 1536).cuda(), g.cuda())
    assert rstd is None and y.shape == (4, 37, 1536)
    check_all(h.view(-1, 1536), y.view(-1, 1536), None, x, r, g, 1e-6, "3-D fp16")
