"""Pins for the oracle's gate/up projection with the fused activation,
h = act(x @ wg^T) * (x @ wu^T) ("Fused Kernels", section 4).

Each pin takes an implementation exposing ``gemm_glu(kind, x, wg, wu,
want_gu=False)`` (the oracle package has it) and returns failure strings.
Sources of truth, none of which is the oracle:
  * torch's own float64 activations (F.silu, F.gelu, F.gelu(tanh), F.relu)
    and numpy's matmul (library routines);
  * one-hot rows of x, which turn the products into a lookup of weight
    columns and the whole op into the elementwise activation of them;
  * exact rational arithmetic (fractions) for ReLU on small dyadic inputs;
  * invariants: permutations of k, of rows of x and of output features;
    ReLU's homogeneity; linearity in the up weights.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

KINDS = ("silu", "gelu_erf", "gelu_tanh", "relu")


def torch_act(kind, v):
    t = torch.from_numpy(np.asarray(v, np.float64))
    if kind == "silu":
        r = F.silu(t)
    elif kind == "gelu_erf":
        r = F.gelu(t)
    elif kind == "gelu_tanh":
        r = F.gelu(t, approximate="tanh")
    else:
        r = F.relu(t)
    return r.numpy()


# torch evaluates GELU as 0.5*x*(1 + erf(...)) / (1 + tanh(...)), which
# cancels for x << 0 (relative error ~1e-11 at x = -3.5); the oracle's forms
# do not.  Mistakes the pins look for change results at O(1).
RTOL_TORCH = {"silu": 1e-15, "gelu_erf": 1e-9, "gelu_tanh": 1e-9, "relu": 0.0}


def _fail(name, got, want, rtol, atol=0.0):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if got.shape != want.shape:
        return [f"{name}: shape {got.shape} != {want.shape}"]
    bad = ~(np.abs(got - want) <= atol + rtol * np.abs(want))
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        return [f"{name}: {int(bad.sum())} mismatches, first at {i}: got {got.flat[i]!r} want {want.flat[i]!r}"]
    return []


def _weights(N, K, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(0, 1.5, (N, K)), rng.normal(0, 1, (N, K))


def pin_one_hot_rows(impl):
    """x = the K x K identity: g[m][n] = wg[n][m], u[m][n] = wu[n][m], so h is
    the elementwise activation of the weights' columns (torch's activations).
    N != K so a transposed weight cannot pass by shape."""
    f = []
    K, N = 6, 5
    wg, wu = _weights(N, K, 1)
    x = np.eye(K)
    for kind in KINDS:
        h, g, u = impl.gemm_glu(kind, x, wg, wu, want_gu=True)
        f += _fail(f"{kind} one-hot g", g, wg.T, 0.0)
        f += _fail(f"{kind} one-hot u", u, wu.T, 0.0)
        f += _fail(f"{kind} one-hot h", h, torch_act(kind, wg.T) * wu.T, RTOL_TORCH[kind], 1e-300)
    return f


def pin_k1_is_elementwise(impl):
    """K = 1 with wg = 1: g[m][n] = x[m], u[m][n] = x[m] * wu[n]."""
    f = []
    x = np.array([[-3.5], [-0.75], [0.0], [0.5], [2.25], [40.0]])
    wg = np.ones((4, 1))
    wu = np.array([[1.0], [-2.0], [0.125], [3.0]])
    for kind in KINDS:
        h = impl.gemm_glu(kind, x, wg, wu)
        want = torch_act(kind, np.repeat(x, 4, axis=1)) * (x * wu.T)
        f += _fail(f"{kind} K=1", h, want, RTOL_TORCH[kind], 1e-300)
    return f


def pin_relu_exact_rational(impl):
    """ReLU on dyadic inputs in [-2, 2] with step 1/8: fp64 sums of these
    products are exact, so h must equal the rational result exactly."""
    rng = np.random.default_rng(7)
    M, N, K = 3, 4, 5
    x = rng.integers(-16, 17, (M, K)) / 8
    wg = rng.integers(-16, 17, (N, K)) / 8
    wu = rng.integers(-16, 17, (N, K)) / 8
    want = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            g = sum(Fraction(x[m, k]) * Fraction(wg[n, k]) for k in range(K))
            u = sum(Fraction(x[m, k]) * Fraction(wu[n, k]) for k in range(K))
            want[m, n] = float(max(g, Fraction(0)) * u)
    return _fail("relu exact", impl.gemm_glu("relu", x, wg, wu), want, 0.0)


def pin_library_matmul(impl):
    """g, u against numpy's float64 matmul; h against torch's activation of
    them (bounds: fp64 summation error relative to sum |x w|)."""
    f = []
    rng = np.random.default_rng(11)
    M, N, K = 7, 9, 33
    x = rng.normal(0, 1, (M, K))
    wg, wu = _weights(N, K, 12)
    gm, um = x @ wg.T, x @ wu.T
    scale_g = np.abs(x) @ np.abs(wg).T
    scale_u = np.abs(x) @ np.abs(wu).T
    for kind in KINDS:
        h, g, u = impl.gemm_glu(kind, x, wg, wu, want_gu=True)
        f += _fail(f"{kind} g vs numpy", g, gm, 0.0, 1e-13 * scale_g.max())
        f += _fail(f"{kind} u vs numpy", u, um, 0.0, 1e-13 * scale_u.max())
        f += _fail(f"{kind} h vs torch act", h, torch_act(kind, gm) * um, 1e-12, 1e-12 * (scale_g * scale_u).max())
    return f


def pin_invariants(impl):
    """Permuting k (x's columns with the weights' columns) changes nothing
    beyond rounding; permuting x's rows permutes h's rows; permuting output
    features (wg and wu rows together) permutes h's columns; ReLU is
    homogeneous of degree 2 in x; h is linear in wu."""
    f = []
    rng = np.random.default_rng(5)
    M, N, K = 6, 8, 20
    x = rng.normal(0, 1, (M, K))
    wg, wu = _weights(N, K, 6)
    for kind in KINDS:
        h = impl.gemm_glu(kind, x, wg, wu)
        pk = rng.permutation(K)
        f += _fail(f"{kind} k permutation", impl.gemm_glu(kind, x[:, pk], wg[:, pk], wu[:, pk]), h, 1e-12, 1e-12)
        pm = rng.permutation(M)
        f += _fail(f"{kind} row permutation", impl.gemm_glu(kind, x[pm], wg, wu), h[pm], 0.0)
        pn = rng.permutation(N)
        f += _fail(f"{kind} feature permutation", impl.gemm_glu(kind, x, wg[pn], wu[pn]), h[:, pn], 0.0)
        f += _fail(f"{kind} linear in wu", impl.gemm_glu(kind, x, wg, 4.0 * wu), 4.0 * h, 0.0)
    h = impl.gemm_glu("relu", x, wg, wu)
    f += _fail("relu homogeneity", impl.gemm_glu("relu", 2.0 * x, wg, wu), 4.0 * h, 0.0)
    return f


ALL_PINS = [pin_one_hot_rows, pin_k1_is_elementwise, pin_relu_exact_rational, pin_library_matmul, pin_invariants]


def run_all(impl, pins=ALL_PINS):
    out = []
    for p in pins:
        try:
            out += [f"[{p.__name__}] {m}" for m in p(impl)]
        except Exception as e:
            out.append(f"[{p.__name__}] raised {type(e).__name__}: {e}")
    return out
