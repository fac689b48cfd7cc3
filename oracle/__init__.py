"""fp64 CPU oracle for the fused gated activation (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``mlp_gated_activation_amd`` and never imports it.

The arithmetic lives in ``glu_oracle.c`` (plain scalar C, IEEE double, host
libm).  This module only loads that library, marshals numpy arrays and
applies the ``[gate | up]`` layout, which is pure slicing:

* "Write a Triton SiLU-Mul (SwiGLU) Kernel" -- "Inputs the agent should
  gather first", item 4, and "Correctness requirements": a fused
  ``(rows, 2*I)`` tensor holds the gate ``a`` in its first ``I`` columns and
  the up projection ``b`` in the last ``I``; the activation goes on ``a``.
* "Kernel Profile: SwiGLU (Tier 1 -- Element-wise)" -- "Key Patterns": the
  backward writes ``da, db`` over the saved ``a, b``; in the fused layout the
  gradient is therefore ``dx = [da | db]``.
* "Write a Triton Fused Add+RMSNorm Kernel": ``add_rmsnorm`` below.
* "Fused Kernels", section 4: ``gemm_glu`` below, the gate and up
  projections with the activation applied to their results.

All inputs are the exact values of the stored (already rounded) tensors,
given as float64 arrays; all outputs are unrounded float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

KINDS = {"silu": 0, "gelu_erf": 1, "gelu_tanh": 2, "relu": 3}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "glu_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_lib(force: bool = False) -> str:
    """Compile glu_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build_lib()
        lib = ctypes.CDLL(_LIB)
        d = ctypes.c_double
        i64 = ctypes.c_int64
        pd = ctypes.POINTER(ctypes.c_double)
        lib.oracle_act.argtypes = [ctypes.c_int, d]
        lib.oracle_act.restype = d
        lib.oracle_dact.argtypes = [ctypes.c_int, d]
        lib.oracle_dact.restype = d
        for name in ("oracle_act_n", "oracle_dact_n"):
            getattr(lib, name).argtypes = [ctypes.c_int, i64, pd, pd]
            getattr(lib, name).restype = None
        lib.oracle_fwd.argtypes = [ctypes.c_int, i64, pd, pd, pd]
        lib.oracle_fwd.restype = None
        lib.oracle_bwd.argtypes = [ctypes.c_int, i64, pd, pd, pd, pd, pd]
        lib.oracle_bwd.restype = None
        lib.oracle_add_rmsnorm.argtypes = [i64, i64, pd, pd, pd, d, pd, pd, pd]
        lib.oracle_add_rmsnorm.restype = None
        lib.oracle_gemm_glu.argtypes = [ctypes.c_int, i64, i64, i64, pd, pd, pd, pd, pd, pd]
        lib.oracle_gemm_glu.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def _kind(kind) -> int:
    if isinstance(kind, str):
        return KINDS[kind]
    if int(kind) not in KINDS.values():
        raise ValueError(f"unknown kind {kind!r}")
    return int(kind)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    """OpenMP threads the element loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Sets the OpenMP threads of the element loops (n >= 1)."""
    _load().oracle_set_num_threads(int(n))


def act1(kind, x: float) -> float:
    """act(x) for one scalar."""
    return float(_load().oracle_act(_kind(kind), float(x)))


def dact1(kind, x: float) -> float:
    """act'(x) for one scalar."""
    return float(_load().oracle_dact(_kind(kind), float(x)))


def act(kind, x) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    _load().oracle_act_n(_kind(kind), x.size, _ptr(x), _ptr(out))
    return out


def dact(kind, x) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    _load().oracle_dact_n(_kind(kind), x.size, _ptr(x), _ptr(out))
    return out


def fwd(kind, a, b) -> np.ndarray:
    """y = act(a) * b for separate a, b of one shape."""
    a = _f64(a)
    b = _f64(b)
    if a.shape != b.shape:
        raise ValueError(f"a{a.shape} and b{b.shape} differ in shape")
    y = np.empty_like(a)
    _load().oracle_fwd(_kind(kind), a.size, _ptr(a), _ptr(b), _ptr(y))
    return y


def bwd(kind, a, b, dy):
    """(da, db) = (dy * act'(a) * b, dy * act(a)) for separate a, b, dy."""
    a = _f64(a)
    b = _f64(b)
    dy = _f64(dy)
    if not (a.shape == b.shape == dy.shape):
        raise ValueError("a, b and dy must share one shape")
    da = np.empty_like(a)
    db = np.empty_like(a)
    _load().oracle_bwd(_kind(kind), a.size, _ptr(a), _ptr(b), _ptr(dy), _ptr(da), _ptr(db))
    return da, db


def split_gate_up(x) -> tuple[np.ndarray, np.ndarray]:
    """[gate | up] layout: a = x[:, :I], b = x[:, I:] for x of shape (rows, 2I)."""
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] % 2:
        raise ValueError(f"fused input must be (rows, 2*I), got {x.shape}")
    i = x.shape[1] // 2
    return x[:, :i], x[:, i:]


def fwd_gate_up(kind, x) -> np.ndarray:
    """y = act(x[:, :I]) * x[:, I:]."""
    a, b = split_gate_up(x)
    return fwd(kind, a, b)


def bwd_gate_up(kind, x, dy) -> np.ndarray:
    """dx = [da | db] for the fused layout."""
    a, b = split_gate_up(x)
    da, db = bwd(kind, a, b, dy)
    return np.concatenate([da, db], axis=1)


def add_rmsnorm(x, res, gamma, eps: float):
    """Fused residual add + RMSNorm forward over the last dimension.

    x, res: (rows, H); gamma: (H,).  Returns (h, y, rstd): h = x + res,
    rstd = 1/sqrt(mean(h^2) + eps) per row, y = h * rstd * gamma.
    """
    x = _f64(x)
    res = _f64(res)
    gamma = _f64(gamma)
    if x.ndim != 2 or x.shape != res.shape or gamma.shape != (x.shape[1],):
        raise ValueError("x, res must be (rows, H) and gamma (H,)")
    rows, H = x.shape
    h = np.empty_like(x)
    y = np.empty_like(x)
    rstd = np.empty(rows)
    _load().oracle_add_rmsnorm(rows, H, _ptr(x), _ptr(res), _ptr(gamma), float(eps),
                               _ptr(h), _ptr(y), _ptr(rstd))
    return h, y, rstd


def gemm_glu(kind, x, wg, wu, want_gu: bool = False):
    """h = act(x @ wg^T) * (x @ wu^T) ("Fused Kernels", section 4).

    x: (M, K); wg, wu: (N, K), the [out][in] layout of a linear layer's
    weight.  Returns h (M, N), or (h, g, u) with the pre-activations
    g = x @ wg^T and u = x @ wu^T when want_gu.  fp64 sums in k order.
    """
    x, wg, wu = _f64(x), _f64(wg), _f64(wu)
    if x.ndim != 2 or wg.ndim != 2 or wg.shape != wu.shape or wg.shape[1] != x.shape[1]:
        raise ValueError("x must be (M, K) and wg, wu (N, K)")
    M, K = x.shape
    N = wg.shape[0]
    h = np.empty((M, N))
    g = np.empty((M, N)) if want_gu else None
    u = np.empty((M, N)) if want_gu else None
    null = ctypes.POINTER(ctypes.c_double)()
    _load().oracle_gemm_glu(_kind(kind), M, N, K, _ptr(x), _ptr(wg), _ptr(wu), _ptr(h),
                            _ptr(g) if want_gu else null, _ptr(u) if want_gu else null)
    return (h, g, u) if want_gu else h
