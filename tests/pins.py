"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself.

Each pin takes an implementation object exposing ``act(kind, x)``,
``dact(kind, x)``, ``fwd(kind, a, b)``, ``bwd(kind, a, b, dy)``,
``fwd_gate_up(kind, x)`` and ``bwd_gate_up(kind, x, dy)`` (the ``oracle``
package has exactly this surface) and returns a list of failure strings.
The same pins are run against deliberately broken implementations in
``test_oracle.py`` to show that each plausible mistake is caught.

Sources of truth used here, none of which is the oracle:
  * library routines: scipy.special.expit (logistic), scipy.special.ndtr
    (normal CDF), scipy.special.lambertw, torch CPU float64
    (F.silu, F.gelu, F.relu and autograd), mpmath at 40 digits
    (ncdf, tanh, numerical differentiation, root finding);
  * identities: act(x) - act(-x) = x and act'(x) + act'(-x) = 1;
  * the pages' printed constants and their erf-vs-tanh GELU gap;
  * central differences of the oracle's own forward (the fp64 gradcheck the
    SwiGLU kernel page asks for in "Correctness requirements").
"""
from __future__ import annotations

import math
import os

import mpmath
import numpy as np
import scipy.special as sp
import torch
import torch.nn.functional as F

SMOOTH = ("silu", "gelu_erf", "gelu_tanh")
KINDS = SMOOTH + ("relu",)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    """key = value lines; '#' starts a comment."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("=", 1))
                out[k] = v
    return out


def _rel_fail(name, got, want, rtol, atol=0.0):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bad = ~(err <= atol + rtol * np.abs(want))
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        return [f"{name}: {int(bad.sum())} mismatches, first at {i}: got {got.flat[i]!r} want {want.flat[i]!r}"]
    return []


def sweep16(dtype: torch.dtype, limit: float = 100.0) -> np.ndarray:
    """Every finite value of a 16-bit dtype with |x| <= limit, as float64."""
    v = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(dtype).to(torch.float64).numpy()
    v = v[np.isfinite(v)]
    return np.unique(v[np.abs(v) <= limit])


def grid(lo=-30.0, hi=30.0, n=20001) -> np.ndarray:
    return np.linspace(lo, hi, n)


def cfg0_inputs():
    """The 64x1024 fp32 workload's exact values (a = 2*randn, b, dy = randn)."""
    g = torch.Generator().manual_seed(0)
    a = (torch.randn(64, 1024, generator=g) * 2.0).double().numpy()
    b = torch.randn(64, 1024, generator=g).double().numpy()
    dy = torch.randn(64, 1024, generator=g).double().numpy()
    return a, b, dy


# ----------------------------------------------------------------------------
# P1: closed-form points and library routines
# ----------------------------------------------------------------------------

def pin_zero(impl):
    """act(0) = 0 for every kind; act'(0) = 1/2 for the smooth kinds
    (sigmoid(0) = Phi(0) = 1/2); relu'(0) = 0 (the derivative reading)."""
    f = []
    for k in KINDS:
        if impl.act(k, [0.0])[0] != 0.0:
            f.append(f"act({k})(0) != 0")
    for k in SMOOTH:
        d = impl.dact(k, [0.0])[0]
        if abs(d - 0.5) > 1e-15:
            f.append(f"act'({k})(0) = {d} != 0.5")
    if impl.dact("relu", [0.0])[0] != 0.0:
        f.append("relu'(0) != 0")
    return f


def pin_silu_library(impl):
    """silu(x) = x * expit(x) (scipy's logistic), and against torch's F.silu."""
    x = np.concatenate([grid(-60, 60), sweep16(torch.bfloat16, 80), sweep16(torch.float16, 80)])
    f = _rel_fail("silu vs x*expit(x)", impl.act("silu", x), x * sp.expit(x), 4e-16 * 8, 1e-300)
    t = F.silu(torch.from_numpy(x)).numpy()
    f += _rel_fail("silu vs torch", impl.act("silu", x), t, 1e-14, 1e-300)
    return f


def pin_gelu_erf_library(impl):
    """gelu_erf(x) = x * Phi(x) with scipy's ndtr (tail-accurate normal CDF);
    torch's F.gelu(approximate='none') where 1+erf does not cancel."""
    x = np.concatenate([grid(-35, 35), sweep16(torch.bfloat16, 30), sweep16(torch.float16, 30)])
    # Both sides round x/sqrt2 and evaluate exp(-z^2)-like factors in double,
    # so each carries a relative error of a few (x^2 + 4) ulps in the tail.
    rtol = (x * x + 8.0) * 2.0 ** -52
    f = _rel_fail("gelu_erf vs x*ndtr(x)", impl.act("gelu_erf", x), x * sp.ndtr(x), rtol, 1e-300)
    xt = np.array([-37.5, -30.0, -20.25, -12.0, -7.5, -3.25])
    with mpmath.workdps(40):
        want = np.array([float(v * mpmath.ncdf(v)) for v in xt])
    f += _rel_fail("gelu_erf tail vs mpmath", impl.act("gelu_erf", xt), want,
                   (xt * xt + 8.0) * 2.0 ** -52, 1e-300)
    xs = x[np.abs(x) <= 4]
    t = F.gelu(torch.from_numpy(xs), approximate="none").numpy()
    f += _rel_fail("gelu_erf vs torch", impl.act("gelu_erf", xs), t, 1e-12, 1e-300)
    return f


def _mp_gelu_tanh(x):
    k = mpmath.sqrt(2 / mpmath.pi)
    x = mpmath.mpf(x)
    return 0.5 * x * (1 + mpmath.tanh(k * (x + mpmath.mpf("0.044715") * x ** 3)))


def pin_gelu_tanh_library(impl):
    """tanh-form GELU against torch's F.gelu(approximate='tanh') where 1+tanh
    does not cancel, and against the pages' 0.5*x*(1+tanh(u)) evaluated at
    40 digits by mpmath everywhere (including deep negative tails)."""
    x = np.concatenate([grid(-3, 3, 6001), sweep16(torch.float16, 3)])
    t = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    f = _rel_fail("gelu_tanh vs torch", impl.act("gelu_tanh", x), t, 1e-12, 1e-300)
    xs = np.concatenate([np.linspace(-12, 12, 241), [-20.0, -15.5, 1e-8, -1e-8, 7.25]])
    # 1 + tanh(u) ~ 2 exp(2u) for u << 0: carry enough digits to resolve it
    with mpmath.workdps(400):
        want = np.array([float(_mp_gelu_tanh(v)) for v in xs])
    # relative conditioning of x*sigmoid(2u) in double: about |2u| + 4 ulps
    u2 = np.abs(2 * math.sqrt(2 / math.pi) * (xs + 0.044715 * xs ** 3))
    f += _rel_fail("gelu_tanh vs mpmath", impl.act("gelu_tanh", xs), want,
                   (u2 + 8.0) * 2.0 ** -52, 1e-300)
    return f


def pin_relu(impl):
    """relu(x) = max(x, 0), exact; NaN propagates."""
    x = np.concatenate([grid(-5, 5, 1001), sweep16(torch.bfloat16, 1e30)])
    f = []
    y = impl.act("relu", x)
    if not np.array_equal(y, np.where(x > 0, x, 0.0)):
        f.append("relu(x) != max(x, 0)")
    d = impl.dact("relu", x)
    if not np.array_equal(d, np.where(x > 0, 1.0, 0.0)):
        f.append("relu'(x) != [x > 0]")
    if not np.isnan(impl.act("relu", [np.nan])[0]):
        f.append("relu(NaN) is not NaN")
    return f


# ----------------------------------------------------------------------------
# P2: limits and derivative roots
# ----------------------------------------------------------------------------

def pin_limits(impl):
    """act(x) -> x as x -> +inf and -> 0 from below as x -> -inf."""
    f = []
    for k in KINDS:
        hi = impl.act(k, [40.0, 1e6, 1e30])
        if not np.array_equal(hi, [40.0, 1e6, 1e30]):
            f.append(f"{k}: act(x) != x for large x: {hi}")
        lo = impl.act(k, [-40.0, -1e6, -1e30])
        if np.any(lo > 0) or np.any(np.abs(lo) > 1e-15):
            f.append(f"{k}: act(x) not ~0- for very negative x: {lo}")
    # the leading tail term of silu: silu(-x) ~ -x*exp(-x)
    f += _rel_fail("silu tail", impl.act("silu", [-40.0, -80.0]),
                   [-40 * math.exp(-40) / (1 + math.exp(-40)), -80 * math.exp(-80)], 1e-14)
    return f


def _bisect_root(fn, lo, hi, iters=200):
    flo = fn(lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        fm = fn(mid)
        if (fm < 0) == (flo < 0):
            lo, flo = mid, fm
        else:
            hi = mid
    return 0.5 * (lo + hi)


def pin_silu_root(impl):
    """silu' vanishes once, at x0 = -1 - W(1/e) (Lambert W), where
    sigmoid(x0) = 1 + 1/x0, hence silu(x0) = x0 + 1."""
    x0 = _bisect_root(lambda x: impl.dact("silu", [x])[0], -2.0, -1.0)
    want = -1.0 - float(sp.lambertw(math.exp(-1)).real)
    f = []
    if abs(x0 - want) > 1e-12:
        f.append(f"silu' root {x0!r} != -1-W(1/e) = {want!r}")
    s = impl.act("silu", [want])[0]
    if abs(s - (want + 1.0)) > 1e-14:
        f.append(f"silu(x0) = {s!r} != x0 + 1 = {want + 1.0!r}")
    return f


def _mp_forward(kind):
    if kind == "silu":
        return lambda x: x / (1 + mpmath.exp(-x))
    if kind == "gelu_erf":
        return lambda x: x * mpmath.ncdf(x)
    if kind == "gelu_tanh":
        return _mp_gelu_tanh
    raise ValueError(kind)


def pin_gelu_roots(impl):
    """The roots of gelu' (both forms) match the roots of mpmath's numerical
    derivative of the 40-digit forward, and the minima match too."""
    f = []
    with mpmath.workdps(40):
        for k, guess in (("gelu_erf", -0.75), ("gelu_tanh", -0.75)):
            fw = _mp_forward(k)
            r = mpmath.findroot(lambda x: mpmath.diff(fw, x), mpmath.mpf(guess))
            x0 = _bisect_root(lambda x: impl.dact(k, [x])[0], -1.0, -0.5)
            if abs(x0 - float(r)) > 1e-12:
                f.append(f"{k}' root {x0!r} != mpmath {float(r)!r}")
            m = impl.act(k, [float(r)])[0]
            if abs(m - float(fw(r))) > 1e-15:
                f.append(f"{k} minimum {m!r} != {float(fw(r))!r}")
    return f


# ----------------------------------------------------------------------------
# P3: invariants
# ----------------------------------------------------------------------------

def pin_invariants(impl):
    """act(x) - act(-x) = x and act'(x) + act'(-x) = 1 (x != 0), all kinds."""
    rng = np.random.default_rng(12345)
    x = np.concatenate([rng.normal(0, 3, 20000), sweep16(torch.float16, 60), sweep16(torch.bfloat16, 60)])
    x = x[x != 0]
    f = []
    for k in KINDS:
        d = impl.act(k, x) - impl.act(k, -x)
        f += _rel_fail(f"{k}: act(x)-act(-x)=x", d, x, 4 * 2.0 ** -52)
        s = impl.dact(k, x) + impl.dact(k, -x)
        # the plain definitions carry an absolute error of about |x| ulps
        # (x times a rounded 1 - sigmoid or Phi); allow 4x that
        f += _rel_fail(f"{k}: act'(x)+act'(-x)=1", s, np.ones_like(s), 0.0,
                       4 * (np.abs(x) * x * x / (1 + x * x) + 4) * 2.0 ** -52)
    return f


# ----------------------------------------------------------------------------
# P4: the pages' printed constants and GELU gap
# ----------------------------------------------------------------------------

def pin_erf_tanh_gap(impl):
    """The largest |gelu_erf - gelu_tanh| rounds to the pages' stated figure."""
    g = read_golden("pages_constants.txt")
    stated = float(g["gelu_erf_tanh_max_abs_gap"])
    x = np.linspace(-8, 8, 160001)
    gap = np.max(np.abs(impl.act("gelu_erf", x) - impl.act("gelu_tanh", x)))
    # "~5e-4": the true gap must round to 5e-4 at one significant digit
    if not (0.9 * stated <= gap < 1.1 * stated):
        return [f"max |gelu_erf - gelu_tanh| = {gap:.4g}, pages state ~{stated:g}"]
    return []


# ----------------------------------------------------------------------------
# P5: central differences (fp64 gradcheck) and mpmath derivatives
# ----------------------------------------------------------------------------

def pin_central_differences(impl):
    """d/da and d/db of fwd (times dy) against bwd on the 64x1024 workload."""
    a, b, dy = cfg0_inputs()
    f = []
    h = 2.0 ** -20 * np.maximum(1.0, np.abs(a))
    hb = 2.0 ** -20 * np.maximum(1.0, np.abs(b))
    for k in KINDS:
        da, db = impl.bwd(k, a, b, dy)
        fd_a = (impl.fwd(k, a + h, b) - impl.fwd(k, a - h, b)) / (2 * h) * dy
        fd_b = (impl.fwd(k, a, b + hb) - impl.fwd(k, a, b - hb)) / (2 * hb) * dy
        m = np.ones(a.shape, bool) if k != "relu" else np.abs(a) > 2 * h
        scale = np.abs(dy * b) + 1e-300
        err = np.abs(fd_a - da)[m] / scale[m]
        if not np.all(err <= 1e-7):
            f.append(f"{k}: da vs central difference, max scaled err {err.max():.3g}")
        sc = np.abs(dy) * (np.abs(impl.act(k, a)) + 1e-300)
        errb = np.abs(fd_b - db) / sc
        if not np.all(errb <= 1e-7):
            f.append(f"{k}: db vs central difference, max scaled err {errb.max():.3g}")
    return f


def pin_derivative_mpmath(impl):
    """act'(x) against mpmath's numerical derivative of the 40-digit forward,
    at points that include the derivative's root and deep tails."""
    xs = np.concatenate([np.linspace(-9, 9, 73), [-1.2784, -0.7518, -0.7525, 1e-6, -30.0, 25.0]])
    f = []
    with mpmath.workdps(40):
        for k in SMOOTH:
            fw = _mp_forward(k)
            want = np.array([float(mpmath.diff(fw, mpmath.mpf(v))) for v in xs])
            f += _rel_fail(f"{k}' vs mpmath.diff", impl.dact(k, xs), want, 1e-13, 1e-16)
    return f


def pin_torch_autograd(impl):
    """act' against torch float64 autograd over 16-bit grids."""
    f = []
    for k, lim in (("silu", 60), ("gelu_erf", 4), ("gelu_tanh", 3), ("relu", 60)):
        x = sweep16(torch.float16, lim)
        x = x[x != 0]
        t = torch.from_numpy(x).requires_grad_(True)
        y = {"silu": F.silu, "relu": F.relu,
             "gelu_erf": lambda v: F.gelu(v, approximate="none"),
             "gelu_tanh": lambda v: F.gelu(v, approximate="tanh")}[k](t)
        (g,) = torch.autograd.grad(y.sum(), t)
        f += _rel_fail(f"{k}' vs torch autograd", impl.dact(k, x), g.numpy(), 1e-12, 1e-15)
    return f


# ----------------------------------------------------------------------------
# Layout and backward structure
# ----------------------------------------------------------------------------

def pin_structure(impl):
    """fwd applies act to a (not b); bwd gives da = dy*act'(a)*b and
    db = dy*act(a); the [gate | up] layout takes a from the first half."""
    f = []
    rng = np.random.default_rng(7)
    a = rng.normal(0, 2, (3, 5))
    b = rng.normal(0, 1, (3, 5)) + 3.0      # keep b away from a's distribution
    dy = rng.normal(0, 1, (3, 5))
    for k in KINDS:
        y = impl.fwd(k, a, np.ones_like(a))
        f += _rel_fail(f"{k}: fwd(a, 1) != act(a)", y, impl.act(k, a), 0.0)
        da, db = impl.bwd(k, a, np.ones_like(a), np.ones_like(a))
        f += _rel_fail(f"{k}: bwd(a,1,1).da != act'(a)", da, impl.dact(k, a), 0.0)
        f += _rel_fail(f"{k}: bwd(a,1,1).db != act(a)", db, impl.act(k, a), 0.0)
        da2, _ = impl.bwd(k, a, b, np.ones_like(a))
        f += _rel_fail(f"{k}: da scales with b", da2, impl.dact(k, a) * b, 1e-15)
        _, db2 = impl.bwd(k, a, b, dy)
        f += _rel_fail(f"{k}: db scales with dy", db2, impl.act(k, a) * dy, 1e-15)
        x = np.concatenate([a, np.ones_like(a)], axis=1)
        f += _rel_fail(f"{k}: [gate|up] y != act(gate)", impl.fwd_gate_up(k, x), impl.act(k, a), 0.0)
        dx = impl.bwd_gate_up(k, np.concatenate([a, b], axis=1), dy)
        f += _rel_fail(f"{k}: [gate|up] dx left != da", dx[:, :5], dy * impl.dact(k, a) * b, 1e-15)
        f += _rel_fail(f"{k}: [gate|up] dx right != db", dx[:, 5:], dy * impl.act(k, a), 1e-15)
    return f


def pin_page_constants(impl):
    """The pages print 1/sqrt(2) = 0.7071067811865475 and the tanh-form
    constants sqrt(2/pi) and 0.044715; the forward at x where the constants
    matter most agrees with those exact constants through library routines."""
    g = read_golden("pages_constants.txt")
    c = float(g["inv_sqrt2"])
    f = []
    if c != 1 / math.sqrt(2):
        f.append("page constant 0.7071067811865475 is not 1/sqrt(2) in double")
    x = np.array([-3.0, -1.0, 0.5, 2.0])
    f += _rel_fail("gelu_erf via erfc with the page constant", impl.act("gelu_erf", x),
                   0.5 * x * sp.erfc(-x * c), 1e-14)
    k = math.sqrt(2 / math.pi)
    c3 = float(g["gelu_tanh_cubic"])
    xs = np.array([-2.0, -0.5, 0.7, 2.5])
    want = 0.5 * xs * (1 + np.tanh(k * (xs + c3 * xs ** 3)))
    f += _rel_fail("gelu_tanh with the page constants", impl.act("gelu_tanh", xs), want, 1e-13)
    return f


ALL_PINS = [pin_zero, pin_silu_library, pin_gelu_erf_library, pin_gelu_tanh_library,
            pin_relu, pin_limits, pin_silu_root, pin_gelu_roots, pin_invariants,
            pin_erf_tanh_gap, pin_central_differences, pin_derivative_mpmath,
            pin_torch_autograd, pin_structure, pin_page_constants]


def run_all(impl, pins=ALL_PINS):
    out = []
    for p in pins:
        try:
            out += [f"[{p.__name__}] {m}" for m in p(impl)]
        except Exception as e:  # a broken implementation may also crash a pin
            out.append(f"[{p.__name__}] raised {type(e).__name__}: {e}")
    return out
