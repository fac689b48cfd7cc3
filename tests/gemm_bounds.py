"""Error bound for the gate/up projection with the fused activation,
derived from the arithmetic (used by the GPU parity tests).

The GPU accumulates g = sum_k x_k wg_k and u = sum_k x_k wu_k in fp32 on the
matrix cores (products of 16-bit inputs are exact in fp32), evaluates
act(g) * u in fp32 and rounds h once to the storage type.  With u32 = 2^-24,
any order of K fp32 additions is within
    E_g = gamma_K * sum_k |x_k wg_k|,   gamma_K = K u32 / (1 - K u32)
of the exact g (the standard summation bound), and likewise E_u.  So, with
L = 1.13 >= max |act'| over all four activations (SiLU 1.0998, GELU-erf
1.1289, GELU-tanh 1.1295, ReLU 1),
    |h_gpu - h| <= ulp_T(h) + L E_g (|u| + E_u) + |act(g)| E_u + 2^-13 |act(g) u|
where the last term covers the fp32 evaluation of act and of the product
(the forward GELU-erf's normal CDF is a polynomial fit to 6.5e-5 relative,
the other activations are within a few fp32 ulp), and ulp_T(h) the final
rounding (one output ulp, as for the elementwise kernels).  The pre-activations written to gu satisfy
|g_gpu - g| <= ulp_T(g) + E_g, and the same for u.

The bound is a worst case: typical accumulation errors grow like sqrt(K)
u32, far below one bf16/fp16 ulp, so the tests also report how many
results sit within one output ulp.
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
    return (ulp(h_ref, FORMATS[fmt]) + L_ACT * Eg * (np.abs(u_ref) + Eu) + np.abs(act_g) * Eu
            + 2.0 ** -13 * np.abs(act_g * u_ref))


def pre_bound(fmt: str, K: int, x, w, ref):
    return ulp(ref, FORMATS[fmt]) + gamma(K) * sums_abs(x, w)
