"""Pins for the oracle's fused residual add + RMSNorm forward.

Each pin takes an implementation exposing ``add_rmsnorm(x, res, gamma, eps)
-> (h, y, rstd)`` (the oracle package has it) and returns failure strings.
Sources of truth, none of which is the oracle:
  * torch's own float64 ``torch.nn.functional.rms_norm`` (library routine);
  * closed forms for constant rows and two-valued rows;
  * invariants: mean((y/gamma)^2) = ms/(ms+eps) per row, homogeneity
    y(kx, kr; k^2 eps) = y(x, r; eps), column-permutation equivariance,
    row independence;
  * the page's own numbers where it gives them ("Write a Triton Fused
    Add+RMSNorm Kernel", Correctness requirements: the variance denominator
    is H, eps is inside the square root, gamma is indexed by column only).
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _fail(name, got, want, rtol, atol=0.0):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    bad = ~(np.abs(got - want) <= atol + rtol * np.abs(want))
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        return [f"{name}: {int(bad.sum())} mismatches, first at {i}: got {got.flat[i]!r} want {want.flat[i]!r}"]
    return []


def _inputs(rows=7, H=96, seed=3, res_scale=0.5):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (rows, H))
    r = rng.normal(0, res_scale, (rows, H))
    g = 1.0 + 0.25 * rng.normal(0, 1, H)
    return x, r, g


def pin_torch_rms_norm(impl):
    """y against torch float64 F.rms_norm of h = x + r with the same gamma and
    eps, for several eps (including one large enough to matter)."""
    f = []
    x, r, g = _inputs()
    for eps in (1e-6, 1e-2, 0.5):
        h, y, rstd = impl.add_rmsnorm(x, r, g, eps)
        want = F.rms_norm(torch.from_numpy(x + r), (x.shape[1],), weight=torch.from_numpy(g), eps=eps).numpy()
        f += _fail(f"y vs torch rms_norm (eps={eps})", y, want, 1e-13)
        f += _fail("h = x + r", h, x + r, 0.0)
    return f


def pin_closed_forms(impl):
    """Constant row c: rstd = 1/sqrt(c^2 + eps); row of +a/-a pairs: same with a.
    Zero row: y = 0, rstd = 1/sqrt(eps)."""
    f = []
    H, eps = 64, 1e-3
    g = np.linspace(0.5, 1.5, H)
    c = 1.75
    x = np.full((3, H), c)
    x[1, ::2], x[1, 1::2] = 2.5, -2.5
    x[2, :] = 0.0
    r = np.zeros_like(x)
    h, y, rstd = impl.add_rmsnorm(x, r, g, eps)
    want_rstd = np.array([1 / np.sqrt(c * c + eps), 1 / np.sqrt(6.25 + eps), 1 / np.sqrt(eps)])
    f += _fail("closed-form rstd", rstd, want_rstd, 1e-15)
    f += _fail("closed-form y (constant row)", y[0], c * g / np.sqrt(c * c + eps), 1e-15)
    f += _fail("closed-form y (zero row)", y[2], np.zeros(H), 0.0)
    return f


def pin_invariants(impl):
    """mean((y/gamma)^2) = ms/(ms + eps); homogeneity; permutation
    equivariance over columns; rows are independent."""
    f = []
    x, r, g = _inputs(rows=5, H=200, seed=9)
    eps = 0.05
    h, y, rstd = impl.add_rmsnorm(x, r, g, eps)
    ms = np.mean((x + r) ** 2, axis=1)
    f += _fail("mean((y/g)^2) = ms/(ms+eps)", np.mean((y / g) ** 2, axis=1), ms / (ms + eps), 1e-13)
    k = 3.0
    _, yk, _ = impl.add_rmsnorm(k * x, k * r, g, k * k * eps)
    f += _fail("homogeneity", yk, y, 1e-13)
    p = np.random.default_rng(1).permutation(x.shape[1])
    _, yp, _ = impl.add_rmsnorm(x[:, p], r[:, p], g[p], eps)
    f += _fail("column permutation", yp, y[:, p], 1e-13)
    _, y1, r1 = impl.add_rmsnorm(x[2:3], r[2:3], g, eps)
    f += _fail("row independence", y1[0], y[2], 1e-15)
    f += _fail("row independence rstd", r1, rstd[2:3], 1e-15)
    return f


ALL_PINS = [pin_torch_rms_norm, pin_closed_forms, pin_invariants]


def run_all(impl, pins=ALL_PINS):
    out = []
    for p in pins:
        try:
            out += [f"[{p.__name__}] {m}" for m in p(impl)]
        except Exception as e:
            out.append(f"[{p.__name__}] raised {type(e).__name__}: {e}")
    return out
