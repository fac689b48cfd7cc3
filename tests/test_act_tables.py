"""The normal-CDF tables the GELU-erf kernels evaluate (csrc/glu_erfc.h).

The header is written by csrc/gen_erfc.py from mpmath values; here each table
is checked against scipy's erfcx, an independent implementation, on a dense
grid: Q(t) = erfcx(z) / t with z = 2 (1 - t) / t, i.e. t = 1 / (1 + z / 2)
("Write a Triton SiLU-Mul (SwiGLU) Kernel", reasoning step 7: GELU-erf is
x * Phi(x), Phi(x) = erfc(-x / sqrt 2) / 2).  Horner in t with the stored
coefficients, in float64, as the kernels evaluate it.
"""
from __future__ import annotations

import os
import re

import numpy as np
import pytest
from scipy.special import erfcx

HEADER = os.path.join(os.path.dirname(__file__), "..", "mlp_gated_activation_amd", "csrc", "glu_erfc.h")


def tables():
    text = open(HEADER).read()
    out = {}
    for name in ("Q", "QF", "QD", "QDF"):
        deg = int(re.search(rf"#define GLU_ERFC_{name}_DEG (\d+)", text).group(1))
        body = re.search(rf"#define GLU_ERFC_{name}_COEFFS \{{([^}}]*)\}}", text).group(1)
        coef = [float(v.strip().rstrip("f")) for v in body.split(",")]
        assert len(coef) == deg + 1, name
        out[name] = np.array(coef)
    return out


def horner(coef, t):
    p = np.zeros_like(t)
    for c in coef[::-1]:
        p = p * t + c
    return p


# the bound each table is held to by the kernels' error budgets
BOUNDS = {"Q": 6.0e-7, "QF": 1.0e-4, "QD": 1.0e-9, "QDF": 2.0e-7}


@pytest.mark.parametrize("name", ["Q", "QF", "QD", "QDF"])
def test_table_matches_erfcx(name):
    coef = tables()[name]
    t = np.concatenate([np.geomspace(1e-7, 1e-2, 2000), np.linspace(1e-2, 1.0, 200001)])
    z = 2.0 * (1.0 - t) / t
    q = erfcx(z) / t
    rel = np.abs(horner(coef, t) / q - 1.0)
    assert rel.max() <= BOUNDS[name], f"{name}: max relative error {rel.max():.3e}"


def test_fp32_tables_are_fp32():
    """The two 16-bit-data tables are evaluated in fp32: their coefficients
    must be exact fp32 values."""
    for name in ("Q", "QF"):
        c = tables()[name]
        assert np.array_equal(c.astype(np.float32).astype(np.float64), c), name


def test_phi_from_table_matches_the_normal_cdf():
    """End to end in float64: Phi(x) from the fp64 table over x in [-14, 14]
    against scipy's ndtr, within 1e-9 relative (a planted wrong constant,
    e.g. t from |x| / 2 instead of |x| / (2 sqrt 2), fails by orders)."""
    from scipy.special import ndtr
    coef = tables()["QD"]
    x = np.linspace(-14.0, 14.0, 100001)
    ax = np.abs(x)
    t = 1.0 / (1.0 + ax * (0.5 / np.sqrt(2.0)))
    h = 0.5 * t * horner(coef, t) * np.exp(-0.5 * ax * ax)
    phi = np.where(x >= 0, 1.0 - h, h)
    ref = ndtr(x)
    assert np.max(np.abs(phi / ref - 1.0)) < 1e-9


TAYLOR = os.path.join(os.path.dirname(__file__), "..", "mlp_gated_activation_amd", "csrc", "glu_taylor.h")


def test_gelu_erf_fp64_root_patch():
    """The fp64 expansion of GELU-erf's derivative Phi(x) + x phi(x) about its
    root (used for fp32 data inside |x - x0| < 1/32), against mpmath at 40
    digits: the root is a root, and the polynomial is within 1e-11 relative
    over the zone."""
    import mpmath as mp
    mp.mp.dps = 40
    text = open(TAYLOR).read()
    hi = float(re.search(r"#define GLU_TAYLOR_GELU_ERF_D_X0_HI (\S+)", text).group(1))
    lo = float(re.search(r"#define GLU_TAYLOR_GELU_ERF_D_X0_LO (\S+)", text).group(1))
    body = re.search(r"#define GLU_TAYLOR_GELU_ERF_D_COEFFS \{([^}]*)\}", text).group(1)
    c = [float(v) for v in body.split(",")]

    def g(x):
        return mp.ncdf(x) + x * mp.npdf(x)

    x0 = mp.mpf(hi) + mp.mpf(lo)
    assert abs(g(x0)) < mp.mpf("1e-30")
    worst = mp.mpf(0)
    for s in np.linspace(-1.0, 1.0, 257):
        d = mp.mpf(float(s)) / 32
        if d == 0:
            continue
        p = sum(mp.mpf(ck) * d ** (k + 1) for k, ck in enumerate(c))
        worst = max(worst, abs(p / g(x0 + d) - 1))
    assert worst < 1e-11, float(worst)


def test_ln2_split_is_the_cody_waite_split():
    """The two-word ln2 of the fp64 exp's argument reduction: L1 is ln2
    truncated to 32 significant bits (so k * L1 is exact for |k| < 2^21) and
    L2 is the rest, rounded to fp64; both derived here from a 200-bit ln2."""
    import mpmath as mp
    mp.mp.prec = 200
    text = open(os.path.join(os.path.dirname(HEADER), "glu_act.h")).read()
    m = re.search(r"kLn2Hi = ([0-9.e+-]+), kLn2Lo = ([0-9.e+-]+);", text)
    hi, lo = float(m.group(1)), float(m.group(2))
    ln2 = mp.log(2)
    assert hi == float(mp.floor(ln2 * 2 ** 32) / 2 ** 32)
    assert lo == float(ln2 - mp.mpf(hi))
    assert np.frexp(hi)[0] * 2 ** 32 == int(np.frexp(hi)[0] * 2 ** 32)   # 32 significant bits
