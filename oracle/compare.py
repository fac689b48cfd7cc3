"""Output-ulp comparator between a stored GPU result and the fp64 oracle.

Test infrastructure only (see the package docstring).

The contract is "within one unit in the last place of the output dtype":

* bf16 / fp16: pass iff ``|g - r| <= ulp_T(r)`` where
  ``ulp_T(r) = 2**(max(floor(log2|r|), emin_T) - p_T + 1)``; in the normal
  range this is a relative bound of 2**-7 (bf16) or 2**-10 (fp16), and the
  ``emin_T`` floor keeps it meaningful for zero and subnormal results.
* fp32: pass iff ``|g - r| <= max(1e-6 * |r|, 2**-149)``.

``g`` is the stored result converted exactly to float64, ``r`` the unrounded
oracle value.  A stored infinity passes when the correctly rounded value
overflows to the same infinity (or is one ulp from it).  A NaN reference
requires a NaN result; a NaN result with a finite reference fails.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fmt:
    name: str
    p: int      # significand bits, hidden bit included
    emin: int   # exponent of the smallest normal
    emax: int   # exponent of the largest finite binade


FORMATS = {
    "bf16": Fmt("bf16", 8, -126, 127),
    "fp16": Fmt("fp16", 11, -14, 15),
    "fp32": Fmt("fp32", 24, -126, 127),
}

_CHUNK = 1 << 22


def ulp(r: np.ndarray, fmt: Fmt) -> np.ndarray:
    """ulp_T(r) with the subnormal floor, for finite r (float64)."""
    ar = np.abs(r)
    _, e = np.frexp(ar)              # ar = m * 2**e, m in [0.5, 1)
    ex = np.where(ar > 0, e - 1, fmt.emin)
    ex = np.maximum(ex, fmt.emin)
    return np.ldexp(1.0, (ex - fmt.p + 1).astype(np.int32))


def _chunk_errors(g: np.ndarray, r: np.ndarray, fmt: Fmt):
    """Return (error in ulps, pass mask) for one chunk."""
    big = np.ldexp(1.0, fmt.emax + 1)                      # first value past max
    ovf = big - np.ldexp(1.0, fmt.emax - fmt.p)            # rounds to inf from here up
    gnan = np.isnan(g)
    rnan = np.isnan(r)
    ginf = np.isinf(g)
    rinf = np.isinf(r)
    gf = np.where(ginf, np.sign(g) * big, g)
    rf = np.where(rinf | rnan, 0.0, r)
    u = ulp(rf, fmt)
    with np.errstate(invalid="ignore"):
        err = np.abs(gf - rf)
    if fmt.name == "fp32":
        tol = np.maximum(1e-6 * np.abs(rf), np.ldexp(1.0, -149))
        ok = err <= tol
    else:
        ok = err <= u
    # stored inf where the correctly rounded value is that same inf
    ok |= ginf & ~rinf & (np.sign(g) * rf >= ovf)
    # non-finite references
    ok = np.where(rinf, g == r, ok)
    ok = np.where(rnan, gnan, ok)
    ok &= ~(gnan & ~rnan)
    with np.errstate(invalid="ignore", divide="ignore"):
        eu = np.where(rinf | rnan, np.where(ok, 0.0, np.inf), err / u)
    eu = np.where(gnan & ~rnan, np.inf, eu)
    return eu, ok


@dataclass
class Report:
    fmt: str
    count: int
    n_fail: int
    max_ulp: float
    argmax: int
    got_at_max: float
    ref_at_max: float

    @property
    def ok(self) -> bool:
        return self.n_fail == 0

    def __str__(self) -> str:
        return (f"{self.fmt}: n={self.count} fail={self.n_fail} max_ulp={self.max_ulp:.4g} "
                f"at flat index {self.argmax} (got {self.got_at_max!r}, exact {self.ref_at_max!r})")


def compare(got, ref, fmt: str) -> Report:
    """Element-by-element comparison of ``got`` (stored values) with ``ref``."""
    f = FORMATS[fmt]
    g = np.asarray(got, dtype=np.float64).reshape(-1)
    r = np.asarray(ref, dtype=np.float64).reshape(-1)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    n = g.size
    if n == 0:
        return Report(fmt, 0, 0, 0.0, 0, 0.0, 0.0)
    n_fail = 0
    best = (False, -1.0)   # (is a failure, error in ulps): failures rank first
    arg = 0
    for s in range(0, n, _CHUNK):
        eu, ok = _chunk_errors(g[s:s + _CHUNK], r[s:s + _CHUNK], f)
        nf = int(np.count_nonzero(~ok))
        n_fail += nf
        if nf:
            i = int(np.argmax(np.where(ok, -1.0, eu)))
        else:
            i = int(np.argmax(eu))
        cand = (nf > 0, float(eu[i]))
        if cand > best:
            best = cand
            arg = s + i
    return Report(fmt, n, n_fail, best[1], arg, float(g[arg]), float(r[arg]))


def assert_within_one_ulp(got, ref, fmt: str, what: str = "") -> Report:
    rep = compare(got, ref, fmt)
    if not rep.ok:
        raise AssertionError(f"{what}: {rep}")
    return rep
