"""CPU tests of the oracle's fused add + RMSNorm: its pins, and planted
mistakes (in numpy copies built here) that each pin set must catch."""
import numpy as np
import pytest

import oracle
import pins_rmsnorm as pins


class Impl:
    def __init__(self, fn):
        self.add_rmsnorm = fn


def _mk(mean_sub=False, eps_outside=False, denom=0, no_gamma=False, stats_on_x=False,
        sqrt_not_rsqrt=False, gamma_rev=False):
    def fn(x, r, g, eps):
        x, r, g = (np.asarray(v, np.float64) for v in (x, r, g))
        h = x + r
        src = x if stats_on_x else h
        if mean_sub:
            src = src - src.mean(axis=1, keepdims=True)
            hh = h - h.mean(axis=1, keepdims=True)
        else:
            hh = h
        H = x.shape[1] + denom
        ms = (src ** 2).sum(axis=1) / H
        rs = 1 / (np.sqrt(ms) + eps) if eps_outside else (np.sqrt(ms + eps) if sqrt_not_rsqrt else 1 / np.sqrt(ms + eps))
        gg = np.ones_like(g) if no_gamma else (g[::-1] if gamma_rev else g)
        return h, hh * rs[:, None] * gg, rs
    return Impl(fn)


MUTANTS = {
    "LayerNorm mean subtraction": _mk(mean_sub=True),
    "eps outside the sqrt": _mk(eps_outside=True),
    "denominator H - 1": _mk(denom=-1),
    "no gamma": _mk(no_gamma=True),
    "statistics on x, not x + r": _mk(stats_on_x=True),
    "sqrt instead of 1/sqrt": _mk(sqrt_not_rsqrt=True),
    "gamma reversed": _mk(gamma_rev=True),
}


def test_oracle_passes_rmsnorm_pins():
    f = pins.run_all(oracle)
    assert f == [], "\n".join(f)


def test_faithful_copy_passes():
    f = pins.run_all(_mk())
    assert f == [], "\n".join(f)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_rmsnorm_pins_catch_planted_mistake(name):
    assert pins.run_all(MUTANTS[name]), f"no pin caught: {name}"


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.add_rmsnorm(np.zeros((2, 3)), np.zeros((2, 4)), np.ones(3), 1e-6)
    with pytest.raises(ValueError):
        oracle.add_rmsnorm(np.zeros((2, 3)), np.zeros((2, 3)), np.ones(4), 1e-6)
