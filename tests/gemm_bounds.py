"""Error bound for the gate/up projection with the fused activation
("Fused Kernels", section 4: gate and up tiles accumulated, the activation
applied in registers), derived from a contract that names no particular
implementation of the activation.

Contract.  g~ and u~ are sums of the K exact products x_k w_k (products of
16-bit inputs are exact in fp32) accumulated in fp32 in any order, and the
epilogue is held to the elementwise kernels' own contract: h_gpu is within
one output ulp of the exact act(g~) * u~.  Nothing else is allowed to err.

Bound.  With u32 = 2^-24, any order of K fp32 additions is within
    E_g = gamma_K * sum_k |x_k wg_k|,   gamma_K = K u32 / (1 - K u32)
of the exact g (the standard summation bound), and likewise E_u for u.
With L = 1.13 >= max |act'| over the four activations (SiLU 1.0998,
GELU-erf 1.1289, GELU-tanh 1.1295, ReLU 1, properties of the functions),
    |act(g~) u~ - act(g) u| <= Delta = L E_g (|u| + E_u) + |act(g)| E_u,
so |act(g~) u~| <= |h| + Delta and, ulp_T being non-decreasing in |x|,
    |h_gpu - h| <= ulp_T(|h| + Delta) + Delta.
The pre-activations written to gu are g~ rounded once:
    |g_gpu - g| <= ulp_T(|g| + E_g) + E_g, and the same for u.

A kernel meets the epilogue contract when its fp32 evaluation of
act(g~) * u~ errs by less than half an output ulp before the final
round-to-nearest: 2^-9 relative for bf16, 2^-12 for fp16.  The bound is a
worst case; typical accumulation errors grow like sqrt(K) u32, so the tests
also report how many results sit within one output ulp of the exact h.
"""
from __future__ import annotations

import numpy as np

from oracle.compare import FORMATS, ulp

L_ACT = 1.13
U32 = 2.0 ** -24


def gamma(K: int) -> float:
    return K * U32 / (1 - K * U32)


def sums_abs(x, w):
    return np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(w, np.float64)).T


def h_bound(fmt: str, K: int, x, wg, wu, h_ref, g_ref, u_ref, act_g):
    Eg = gamma(K) * sums_abs(x, wg)
    Eu = gamma(K) * sums_abs(x, wu)
    delta = L_ACT * Eg * (np.abs(u_ref) + Eu) + np.abs(act_g) * Eu
    return ulp(np.abs(h_ref) + delta, FORMATS[fmt]) + delta


def pre_bound(fmt: str, K: int, x, w, ref):
    E = gamma(K) * sums_abs(x, w)
    return ulp(np.abs(ref) + E, FORMATS[fmt]) + E
