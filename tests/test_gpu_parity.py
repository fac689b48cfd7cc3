"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every comparison is element by element on the same seeded inputs, with the
one-output-ulp bound of oracle/compare.py (bf16 2^-7, fp16 2^-10 relative,
fp32 1e-6 relative, subnormal floor).  ReLU is exact in the arithmetic the
kernels use, so its results must equal the correctly rounded exact value bit
for bit (zeros compare by value: +0 and -0 are the same exact result).  Non-finite inputs are outside the parity contract; for them only
NaN-in -> NaN-out is checked.
"""
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
KINDS = ("silu", "gelu_erf", "gelu_tanh", "relu")


@pytest.fixture(scope="module")
def glu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conftest import ensure_built
    ensure_built()
    from mlp_gated_activation_amd import glu as g   # raises if libglu.so cannot load
    return g


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def check(got: torch.Tensor, ref: np.ndarray, what: str, exact: bool = False):
    """Within one output ulp of the oracle; bit-exact when `exact`."""
    g = f64(got)
    rep = compare(g, ref, FMT[got.dtype])
    assert rep.ok, f"{what}: {rep}"
    if exact:
        want = torch.from_numpy(np.ascontiguousarray(ref)).to(torch.float32).to(got.dtype)
        gb = got.detach().cpu().contiguous().view(-1)
        wb = want.contiguous().view(-1)
        ib = torch.int16 if got.dtype != torch.float32 else torch.int32
        # zeros compare by value: the sign of an exact zero product is not part
        # of the contract (the compiler may round x*y through fma(x, y, +0))
        skip = torch.isnan(wb) | ((wb == 0) & (gb == 0))
        bad = (gb.view(ib) != wb.view(ib)) & ~skip
        assert not bool(bad.any()), f"{what}: {int(bad.sum())} results differ from RNE(exact)"
    return rep


def cuda(*ts):
    return [t.cuda() for t in ts]


# ---------------------------------------------------------------------------
# The workloads at full size
# ---------------------------------------------------------------------------

def _separate_fwd_bwd(glu, kind, a, b, dy, name, bwd_out_of_place=True):
    """fwd out-of-place, bwd out-of-place (fresh buffers), bwd in place."""
    ga, gb, gdy = cuda(a, b, dy)
    y = glu.glu_fwd(kind, "separate", ga, gb)
    fa, fb, fdy = f64(a), f64(b), f64(dy)
    exact = kind == "relu"
    check(y, oracle.fwd(kind, fa, fb), f"{name} {kind} fwd", exact)
    del y
    rda, rdb = oracle.bwd(kind, fa, fb, fdy)
    if bwd_out_of_place:
        da, db = glu.glu_bwd(kind, "separate", ga, gb, gdy, inplace=False)
        check(da, rda, f"{name} {kind} bwd da", exact)
        check(db, rdb, f"{name} {kind} bwd db", exact)
        del da, db
    glu.glu_bwd(kind, "separate", ga, gb, gdy, inplace=True)
    check(ga, rda, f"{name} {kind} bwd in-place da", exact)
    check(gb, rdb, f"{name} {kind} bwd in-place db", exact)


def test_fp32_64x1024_all_kinds(glu):
    w = inputs.WORKLOADS["swiglu_f32_64x1024"]
    a, b, dy = w.make()
    for kind in KINDS:
        _separate_fwd_bwd(glu, kind, a, b, dy, w.name)


def test_bf16_4096x11008(glu):
    w = inputs.WORKLOADS["swiglu_bf16_4096x11008"]
    a, b, dy = w.make()
    _separate_fwd_bwd(glu, "silu", a, b, dy, w.name)


def test_bf16_gate_up_4096x14336(glu):
    w = inputs.WORKLOADS["swiglu_bf16_gateup_4096x14336"]
    x, dy = w.make()
    gx, gdy = cuda(x, dy)
    fx, fdy = f64(x), f64(dy)
    ref = oracle.fwd_gate_up("silu", fx)
    y = glu.glu_fwd("silu", "gate_up", gx)
    check(y, ref, "gate_up fwd out-of-place")
    del y
    gx2 = gx.clone()
    out = glu.glu_fwd("silu", "gate_up", gx2, inplace=True)
    check(out, ref, "gate_up fwd in-place over b")
    assert torch.equal(gx2[:, :w.cols], gx[:, :w.cols]), "in-place forward touched the gate half"
    del gx2, out
    rdx = oracle.bwd_gate_up("silu", fx, fdy)
    dx = glu.glu_bwd("silu", "gate_up", gx, None, gdy, inplace=False)
    check(dx, rdx, "gate_up bwd out-of-place dx")
    del dx
    glu.glu_bwd("silu", "gate_up", gx, None, gdy, inplace=True)
    check(gx, rdx, "gate_up bwd in-place dx")


@pytest.mark.parametrize("name", [f"swiglu_bf16_4096x{h}" for h in (1024, 2048, 4096, 8192, 16384)]
                         + ["swiglu_bf16_tp8_4096x1792"])
def test_bf16_hidden_sweep(glu, name):
    w = inputs.WORKLOADS[name]
    a, b, dy = w.make()
    _separate_fwd_bwd(glu, "silu", a, b, dy, w.name, bwd_out_of_place=False)


@pytest.mark.parametrize("cols", [8184, 8192])
def test_launch_shape_switch(glu, cols):
    """Either side of 2^22 units (4096 x 8192 bf16), where the launcher
    switches the backward from 512- to 128-thread blocks and starts capping
    resident workgroups: fwd and bwd, in place and not, GELU-erf (the longest
    arithmetic) and ReLU (bit-exact)."""
    a, b, dy = inputs.separate(4096, cols, "bf16", 2.0, seed=7)
    for kind in ("gelu_erf", "relu"):
        _separate_fwd_bwd(glu, kind, a, b, dy, f"4096x{cols}")


@pytest.fixture(scope="module")
def stress_inputs():
    w = inputs.WORKLOADS["geglu_reglu_fp16_gateup_8191x18944"]
    x, dy = w.make()
    return w, x, dy, f64(x), f64(dy)


@pytest.mark.parametrize("kind", ["gelu_erf", "gelu_tanh", "relu"])
def test_fp16_gate_up_8191x18944(glu, stress_inputs, kind):
    w, x, dy, fx, fdy = stress_inputs
    gx, gdy = cuda(x, dy)
    exact = kind == "relu"
    y = glu.glu_fwd(kind, "gate_up", gx)
    check(y, oracle.fwd_gate_up(kind, fx), f"{w.name} {kind} fwd", exact)
    del y
    glu.glu_bwd(kind, "gate_up", gx, None, gdy, inplace=True)
    check(gx, oracle.bwd_gate_up(kind, fx, fdy), f"{w.name} {kind} bwd in-place", exact)


def test_headline_bf16_4096x14336(glu):
    """The benchmarked sequence: fwd out-of-place, then bwd in place."""
    w = inputs.WORKLOADS["swiglu_bf16_4096x14336"]
    a, b, dy = w.make()
    ga, gb, gdy = cuda(a, b, dy)
    fa, fb, fdy = f64(a), f64(b), f64(dy)
    y = glu.glu_fwd("silu", "separate", ga, gb)
    glu.glu_bwd("silu", "separate", ga, gb, gdy, inplace=True)
    check(y, oracle.fwd("silu", fa, fb), "headline fwd")
    rda, rdb = oracle.bwd("silu", fa, fb, fdy)
    check(ga, rda, "headline bwd da")
    check(gb, rdb, "headline bwd db")


# ---------------------------------------------------------------------------
# Every 16-bit input, every kind
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("kind", KINDS)
def test_exhaustive_16bit(glu, dtype, kind):
    a = inputs.all_bit_patterns(dtype).reshape(256, 256)
    fa = f64(a)
    finite = np.isfinite(fa)
    nan_in = np.isnan(fa)
    g = torch.Generator().manual_seed(3)
    for label, b, dy in [
        ("b=dy=1", torch.ones_like(a), torch.ones_like(a)),
        ("random b, dy", torch.randn(256, 256, generator=g).to(a.dtype),
         torch.randn(256, 256, generator=g).to(a.dtype)),
    ]:
        ga, gb, gdy = cuda(a, b, dy)
        fb, fdy = f64(b), f64(dy)
        exact = kind == "relu"
        y = glu.glu_fwd(kind, "separate", ga, gb)
        da, db = glu.glu_bwd(kind, "separate", ga, gb, gdy, inplace=False)
        ry = oracle.fwd(kind, fa, fb)
        rda, rdb = oracle.bwd(kind, fa, fb, fdy)
        for got, ref, nm in ((y, ry, "y"), (da, rda, "da"), (db, rdb, "db")):
            gv = f64(got)
            rep = compare(gv[finite], ref[finite], dtype)
            assert rep.ok, f"{dtype} {kind} {label} {nm}: {rep}"
            assert np.all(np.isnan(gv[nan_in])), f"{dtype} {kind} {label} {nm}: NaN input gave non-NaN"
            if exact:
                check(got.cpu()[torch.from_numpy(finite)], ref[finite], f"{dtype} {kind} {label} {nm}", True)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("kind", KINDS)
def test_kind_mismatch_is_caught(glu, dtype, kind):
    """Negative control ("Write a Triton SiLU-Mul (SwiGLU) Kernel", Common
    failure modes: GELU variant mismatch): the output of each kind, over every
    finite 16-bit input, must fail the one-ulp comparison against each OTHER
    kind's oracle, on many elements, forward and backward.  The closest pair,
    GELU erf against tanh, differs by more than one bf16 ulp on 335 of the
    65280 finite bf16 inputs; a kernel that computed the wrong variant, or a
    comparator too loose to see it, fails here."""
    a = inputs.all_bit_patterns(dtype).reshape(-1)
    fa = f64(a)
    finite = np.isfinite(fa)
    one = torch.ones_like(a)
    ga, gone = cuda(a, one)
    y = f64(glu.glu_fwd(kind, "separate", ga, gone))[finite]
    da, _ = glu.glu_bwd(kind, "separate", ga, gone, gone.clone(), inplace=False)
    da = f64(da)[finite]
    fa, f1 = fa[finite], np.ones(int(finite.sum()))
    assert compare(y, oracle.fwd(kind, fa, f1), dtype).ok
    for other in KINDS:
        if other == kind:
            continue
        ry = oracle.fwd(other, fa, f1)
        rda, _ = oracle.bwd(other, fa, f1, f1)
        for got, ref, nm in ((y, ry, "y"), (da, rda, "da")):
            rep = compare(got, ref, dtype)
            assert not rep.ok and rep.n_fail >= 300, \
                f"{dtype} {kind} output passes as {other} ({nm}): {rep}"


@pytest.mark.parametrize("kind", KINDS)
def test_fp32_wide_range(glu, kind):
    """fp32 inputs from 1e-30 to 1e3 in magnitude, both signs, plus zeros,
    subnormals and the points where act' crosses zero."""
    g = torch.Generator().manual_seed(5)
    mag = torch.exp(torch.empty(1 << 16).uniform_(np.log(1e-30), np.log(1e3), generator=g))
    sgn = torch.where(torch.rand(1 << 16, generator=g) < 0.5, -1.0, 1.0)
    a = (mag * sgn).float()
    special = torch.tensor([0.0, -0.0, 1e-45, -1e-45, 1e-40, -1.2784645, -0.7517915, -0.7524614,
                            88.7, -88.7, -103.0, 20.0, -20.0, 1e30, -1e30], dtype=torch.float32)
    a[:special.numel()] = special
    a = a.reshape(256, 256)
    b = torch.randn(256, 256, generator=g)
    dy = torch.randn(256, 256, generator=g)
    ga, gb, gdy = cuda(a, b, dy)
    fa, fb, fdy = f64(a), f64(b), f64(dy)
    exact = kind == "relu"
    check(glu.glu_fwd(kind, "separate", ga, gb), oracle.fwd(kind, fa, fb), f"fp32 {kind} fwd", exact)
    da, db = glu.glu_bwd(kind, "separate", ga, gb, gdy, inplace=False)
    rda, rdb = oracle.bwd(kind, fa, fb, fdy)
    check(da, rda, f"fp32 {kind} da", exact)
    check(db, rdb, f"fp32 {kind} db", exact)


@pytest.mark.parametrize("kind", KINDS)
def test_fp32_dense_sweep(glu, kind):
    """fp32 data is computed in fp64 with a short exp, reciprocal and (GELU-erf
    forward) normal-CDF table: a dense sweep of a over [-120, 120], where the
    results run from overflow-free growth down through the fp32 subnormals to
    zero, against the oracle within 1e-6 relative."""
    n = 1 << 20
    a = torch.linspace(-120.0, 120.0, n, dtype=torch.float64).float()
    # every fp32 value in windows where an exp argument crosses a range edge
    # or the result turns subnormal (silu near -87 .. -104, GELU-erf near -13 .. -14.5)
    wins = [torch.arange(v, v + 4096, dtype=torch.int32).view(torch.float32)
            for v in (int(np.float32(-87.3).view(np.int32)), int(np.float32(-103.9).view(np.int32)),
                      int(np.float32(-13.2).view(np.int32)), int(np.float32(-14.1).view(np.int32)),
                      int(np.float32(0.5).view(np.int32)))]
    # every fp32 value within 2048 ulps of each act' root, and across the
    # edge of the GELU-erf root's Taylor zone (|x - x0| = 1/32)
    for root in (-1.2784645, -0.7517915, -0.7524614, -0.7517915 - 1 / 32, -0.7517915 + 1 / 32):
        c = int(np.float32(root).view(np.int32))
        wins.append(torch.arange(c - 2048, c + 2048, dtype=torch.int32).view(torch.float32))
    a = torch.cat([a] + wins)
    a = a[: (a.numel() // 512) * 512].reshape(-1, 512)
    g = torch.Generator().manual_seed(11)
    for label, b, dy in [("b=dy=1", torch.ones_like(a), torch.ones_like(a)),
                         ("random b, dy", torch.randn(a.shape, generator=g), torch.randn(a.shape, generator=g))]:
        ga, gb, gdy = cuda(a, b, dy)
        fa, fb, fdy = f64(a), f64(b), f64(dy)
        exact = kind == "relu"
        check(glu.glu_fwd(kind, "separate", ga, gb), oracle.fwd(kind, fa, fb), f"fp32 {kind} fwd {label}", exact)
        da, db = glu.glu_bwd(kind, "separate", ga, gb, gdy, inplace=False)
        rda, rdb = oracle.bwd(kind, fa, fb, fdy)
        check(da, rda, f"fp32 {kind} da {label}", exact)
        check(db, rdb, f"fp32 {kind} db {label}", exact)


# ---------------------------------------------------------------------------
# Shapes, strides, alignment, aliasing and canaries
# ---------------------------------------------------------------------------

SENTINEL = {torch.bfloat16: 0x7FA5, torch.float16: 0x7DA5, torch.float32: 0x7FA5A5A5}  # quiet-NaN patterns


def _canvas(rows, ld, width, dtype, col0, extra_rows=2):
    """A sentinel-filled buffer with a (rows, width) view at column col0,
    row stride ld, starting after one padding row."""
    ib = torch.int32 if dtype == torch.float32 else torch.int16
    total = (rows + extra_rows) * ld + 64
    buf = torch.full((total,), SENTINEL[dtype], dtype=ib).view(dtype).cuda()
    start = ld + col0
    view = buf.as_strided((rows, width), (ld, 1), start)
    return buf, view


def _untouched(buf, view, dtype, what):
    ib = torch.int32 if dtype == torch.float32 else torch.int16
    mask = torch.ones(buf.numel(), dtype=torch.bool)
    rows, width = view.shape
    ld = view.stride(0)
    off = view.storage_offset()
    idx = (off + torch.arange(rows)[:, None] * ld + torch.arange(width)[None, :]).reshape(-1)
    mask[idx] = False
    bits = buf.view(ib).cpu()[mask]
    s = SENTINEL[dtype]
    assert bool((bits == s).all()), f"{what}: {int((bits != s).sum())} elements outside the operand changed"


def _fill(view, src):
    view.copy_(src.cuda())


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("layout", ["separate", "gate_up"])
def test_edge_shapes_with_canaries(glu, dtype, layout):
    t = DT[dtype]
    g = torch.Generator().manual_seed(11)
    for cols in (1, 2, 7, 8, 9, 15, 16, 17, 31, 33, 4095):
        for rows in (1, 3):
            for pad in (0, 5, 8):           # row-stride gap; 5 breaks 16-byte alignment
                for kind in KINDS:
                    a = (torch.randn(rows, cols, generator=g) * 2).to(t)
                    b = torch.randn(rows, cols, generator=g).to(t)
                    dy = torch.randn(rows, cols, generator=g).to(t)
                    fa, fb, fdy = f64(a), f64(b), f64(dy)
                    exact = kind == "relu"
                    tag = f"{dtype} {layout} {kind} rows={rows} cols={cols} pad={pad}"
                    ry = oracle.fwd(kind, fa, fb)
                    rda, rdb = oracle.bwd(kind, fa, fb, fdy)
                    if layout == "separate":
                        ld = cols + pad
                        abuf, av = _canvas(rows, ld, cols, t, 0)
                        bbuf, bv = _canvas(rows, ld, cols, t, 0)
                        _fill(av, a)
                        _fill(bv, b)
                        ybuf, yv = _canvas(rows, ld, cols, t, 0)
                        glu.glu_fwd(kind, "separate", av, bv, yv)
                        check(yv, ry, tag + " fwd", exact)
                        _untouched(ybuf, yv, t, tag + " fwd y")
                        dybuf, dyv = _canvas(rows, ld, cols, t, 0)
                        _fill(dyv, dy)
                        glu.glu_bwd(kind, "separate", av, bv, dyv, inplace=True)
                        check(av, rda, tag + " bwd da", exact)
                        check(bv, rdb, tag + " bwd db", exact)
                        _untouched(abuf, av, t, tag + " da")
                        _untouched(bbuf, bv, t, tag + " db")
                    else:
                        ld = 2 * cols + pad
                        xbuf, xv = _canvas(rows, ld, 2 * cols, t, 0)
                        _fill(xv, torch.cat([a, b], 1))
                        ybuf, yv = _canvas(rows, cols + pad, cols, t, 0)
                        glu.glu_fwd(kind, "gate_up", xv, None, yv)
                        check(yv, ry, tag + " fwd", exact)
                        _untouched(ybuf, yv, t, tag + " fwd y")
                        dybuf, dyv = _canvas(rows, cols + pad, cols, t, 0)
                        _fill(dyv, dy)
                        glu.glu_bwd(kind, "gate_up", xv, None, dyv, inplace=True)
                        check(xv, np.concatenate([rda, rdb], 1), tag + " bwd dx", exact)
                        _untouched(xbuf, xv, t, tag + " dx")
                        # in-place forward over the up half, from fresh inputs
                        _fill(xv, torch.cat([a, b], 1))
                        glu.glu_fwd(kind, "gate_up", xv, inplace=True)
                        check(xv[:, cols:], ry, tag + " fwd in-place", exact)
                        _untouched(xbuf, xv, t, tag + " fwd in-place x")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_unaligned_and_strided_views(glu, dtype):
    """Pointers one element past 16-byte alignment (element path) and sliced
    views with wide row strides (vector path), both layouts."""
    t = DT[dtype]
    g = torch.Generator().manual_seed(13)
    rows, cols = 37, 1000
    for kind in KINDS:
        exact = kind == "relu"
        base = (torch.randn(rows, 3 * cols + 24, generator=g) * 2).to(t).cuda()
        dy = torch.randn(rows, cols, generator=g).to(t).cuda()
        for off in (1, 8):                 # 1: unaligned; 8: aligned slice of a wide row
            a = base[:, off:off + cols]
            b = base[:, off + cols + 8:off + 2 * cols + 8]
            fa, fb, fdy = f64(a), f64(b), f64(dy)
            yo = 1 if off == 1 else 8
            y = torch.empty(rows, cols + 16, dtype=t, device="cuda")[:, yo:yo + cols]
            glu.glu_fwd(kind, "separate", a, b, y)
            check(y, oracle.fwd(kind, fa, fb), f"{dtype} {kind} off={off} fwd", exact)
            x = base[:, off:off + 2 * cols]
            fx = f64(x)
            check(glu.glu_fwd(kind, "gate_up", x), oracle.fwd_gate_up(kind, fx),
                  f"{dtype} {kind} off={off} gate_up fwd", exact)
            da, db = glu.glu_bwd(kind, "separate", a, b, dy, inplace=False)
            rda, rdb = oracle.bwd(kind, fa, fb, fdy)
            check(da, rda, f"{dtype} {kind} off={off} da", exact)
            check(db, rdb, f"{dtype} {kind} off={off} db", exact)


def test_exact_alias_is_allowed(glu):
    """An output may be exactly an input: y over a, and the [gate | up]
    halves passed as two separate operands with y over the up half."""
    g = torch.Generator().manual_seed(17)
    a = (torch.randn(64, 512, generator=g) * 2).to(torch.bfloat16)
    b = torch.randn(64, 512, generator=g).to(torch.bfloat16)
    ref = oracle.fwd("silu", f64(a), f64(b))
    ga, gb = cuda(a, b)
    glu.glu_fwd("silu", "separate", ga, gb, ga)
    check(ga, ref, "y over a")
    x = torch.cat([a, b], 1).cuda()
    glu.glu_fwd("silu", "separate", x[:, :512], x[:, 512:], inplace=True)
    check(x[:, 512:], ref, "y over the up half via separate views")
    assert torch.equal(x[:, :512].cpu(), a)


def test_rejections_raise(glu):
    base = torch.zeros(4 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    a = base[:256].view(4, 64)
    y = base[1:257].view(4, 64)                     # overlaps a, shifted by one element
    with pytest.raises(glu.GluError, match="GLU_ERR_ALIAS"):
        glu.glu_fwd("silu", "separate", a, a.clone(), y)
    sq = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        glu.glu_fwd("silu", "separate", sq.t(), sq)  # transposed view: last dim not contiguous
    with pytest.raises(ValueError):
        glu.glu_fwd("swish", "separate", a, a)


def test_zero_sized(glu):
    a = torch.empty(0, 128, dtype=torch.float16, device="cuda")
    assert glu.glu_fwd("silu", "separate", a, a.clone()).shape == (0, 128)
    x = torch.empty(5, 0, dtype=torch.float16, device="cuda")
    assert glu.glu_fwd("gelu_erf", "gate_up", x).shape == (5, 0)


def test_side_stream_ordering(glu):
    """Work enqueued on a non-default stream is ordered on that stream."""
    g = torch.Generator().manual_seed(19)
    a = (torch.randn(512, 4096, generator=g) * 2).to(torch.bfloat16)
    b = torch.randn(512, 4096, generator=g).to(torch.bfloat16)
    dy = torch.randn(512, 4096, generator=g).to(torch.bfloat16)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ga, gb, gdy = cuda(a, b, dy)
        y = glu.glu_fwd("silu", "separate", ga, gb)
        glu.glu_bwd("silu", "separate", ga, gb, gdy, inplace=True)
    s.synchronize()
    fa, fb, fdy = f64(a), f64(b), f64(dy)
    check(y, oracle.fwd("silu", fa, fb), "side stream fwd")
    rda, rdb = oracle.bwd("silu", fa, fb, fdy)
    check(ga, rda, "side stream da")
    check(gb, rdb, "side stream db")


def test_launch_chunking_beyond_2_30_units(glu):
    """More than 2^30 16-byte units: the dense path splits one long row into
    column chunks and the gate_up path splits rows; sampled outputs (around
    every chunk boundary, the tail and random points) against the oracle."""
    gen = torch.Generator(device="cuda").manual_seed(23)
    n = (1 << 33) + (1 << 20) + 3            # bf16 elements: 2^30 + 2^17 + 1 units
    a = torch.randn(n, device="cuda", dtype=torch.bfloat16, generator=gen)
    b = torch.randn(n, device="cuda", dtype=torch.bfloat16, generator=gen)
    y = glu.glu_fwd("silu", "separate", a, b)
    torch.cuda.synchronize()
    idx = torch.cat([torch.arange(0, 64), torch.arange((1 << 33) - 64, (1 << 33) + 64), torch.arange(n - 64, n),
                     torch.randint(0, n, (1 << 20,), generator=torch.Generator().manual_seed(1))]).cuda()
    check(y[idx], oracle.fwd("silu", f64(a[idx]), f64(b[idx])), "dense 2^33+ fwd")
    del a, b, y
    torch.cuda.empty_cache()
    rows, cols = (1 << 17) + 3, 1 << 16      # 8192 units per row: 2^30 + 24576 units
    x = torch.randn(rows, 2 * cols, device="cuda", dtype=torch.bfloat16, generator=gen)
    y = glu.glu_fwd("silu", "gate_up", x)
    torch.cuda.synchronize()
    r = torch.cat([torch.tensor([0, (1 << 17) - 1, 1 << 17, rows - 1]),
                   torch.randint(0, rows, (1024,), generator=torch.Generator().manual_seed(2))]).cuda()
    xs = x[r]
    check(y[r], oracle.fwd_gate_up("silu", f64(xs)), "gate_up rows-chunked fwd")
    del x, y, xs
    torch.cuda.empty_cache()


def test_hip_graph_capture_and_replay(glu):
    """The launches capture into a HIP graph (the library allocates nothing
    and issues no memset).  Several replays, with eager work and new inputs
    between them; every replay equals the eager result bit for bit."""
    R, C = 1024, 3000
    t = torch.bfloat16
    a_s = torch.empty(R, C, dtype=t, device="cuda")
    b_s = torch.empty_like(a_s)
    dy_s = torch.empty_like(a_s)
    y_s = torch.empty_like(a_s)
    da_s = torch.empty_like(a_s)
    db_s = torch.empty_like(a_s)
    x_s = torch.empty(R, 2 * C, dtype=t, device="cuda")
    y2_s = torch.empty_like(a_s)
    g = torch.Generator(device="cuda").manual_seed(29)

    def refill():
        a_s.copy_(torch.randn(R, C, device="cuda", generator=g) * 2)
        b_s.copy_(torch.randn(R, C, device="cuda", generator=g))
        dy_s.copy_(torch.randn(R, C, device="cuda", generator=g))
        x_s.copy_(torch.randn(R, 2 * C, device="cuda", generator=g))

    refill()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        glu.glu_fwd("silu", "separate", a_s, b_s, y_s)
        glu.glu_bwd("gelu_tanh", "separate", a_s, b_s, dy_s, da_s, db_s, inplace=False)
        glu.glu_fwd("gelu_erf", "gate_up", x_s, None, y2_s)
    for rep in range(4):
        refill()
        graph.replay()
        torch.cuda.synchronize()
        ey = glu.glu_fwd("silu", "separate", a_s, b_s)
        eda, edb = glu.glu_bwd("gelu_tanh", "separate", a_s, b_s, dy_s, inplace=False)
        ey2 = glu.glu_fwd("gelu_erf", "gate_up", x_s)
        torch.cuda.synchronize()
        for got, want, nm in ((y_s, ey, "y"), (da_s, eda, "da"), (db_s, edb, "db"), (y2_s, ey2, "gate_up y")):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {rep}: {nm} differs from eager"
    # and the eager results themselves are right
    check(y_s, oracle.fwd("silu", f64(a_s), f64(b_s)), "graph replay fwd vs oracle")
