"""CPU tests of the fp64 oracle: its pins, and proof that the pins catch
plausible mistakes (each mistake is planted in a copy of the oracle built
here, on the CPU; the oracle itself is never modified)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special as sp

import oracle
import pins

K = math.sqrt(2 / math.pi)
C3 = 0.044715


class Impl:
    """An implementation assembled from act/dact with the same surface as
    the oracle package; its forward and backward follow the definitions
    y = act(a)*b, da = dy*act'(a)*b, db = dy*act(a)."""

    def __init__(self, act=None, dact=None, swap_grads=False, act_on_b=False,
                 drop_dy_db=False, swap_halves=False):
        self._act = act or {}
        self._dact = dact or {}
        self.swap_grads = swap_grads
        self.act_on_b = act_on_b
        self.drop_dy_db = drop_dy_db
        self.swap_halves = swap_halves

    def act(self, k, x):
        x = np.asarray(x, dtype=np.float64)
        return self._act[k](x) if k in self._act else oracle.act(k, x)

    def dact(self, k, x):
        x = np.asarray(x, dtype=np.float64)
        return self._dact[k](x) if k in self._dact else oracle.dact(k, x)

    def fwd(self, k, a, b):
        a = np.asarray(a, np.float64)
        b = np.asarray(b, np.float64)
        return self.act(k, b) * a if self.act_on_b else self.act(k, a) * b

    def bwd(self, k, a, b, dy):
        a, b, dy = (np.asarray(v, np.float64) for v in (a, b, dy))
        da = dy * self.dact(k, a) * b
        db = (1.0 if self.drop_dy_db else dy) * self.act(k, a)
        return (db, da) if self.swap_grads else (da, db)

    def _split(self, x):
        a, b = oracle.split_gate_up(x)
        return (b, a) if self.swap_halves else (a, b)

    def fwd_gate_up(self, k, x):
        return self.fwd(k, *self._split(x))

    def bwd_gate_up(self, k, x, dy):
        da, db = self.bwd(k, *self._split(x), dy)
        return np.concatenate([da, db], axis=1)


def _sig(x):
    return sp.expit(x)


def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


MUTANTS = {
    "silu uses sigmoid(-x)": Impl(act={"silu": lambda x: x * _sig(-x)}),
    "silu' drops the x(1-s) term": Impl(dact={"silu": _sig}),
    "silu' uses s for 1-s": Impl(dact={"silu": lambda x: _sig(x) * (1 + x * _sig(x))}),
    "gelu_erf drops the 0.5": Impl(act={"gelu_erf": lambda x: x * sp.erfc(-x / math.sqrt(2))}),
    "gelu_erf uses sqrt2 for 1/sqrt2": Impl(act={"gelu_erf": lambda x: 0.5 * x * sp.erfc(-x * math.sqrt(2))}),
    "gelu_erf via 1+erf (cancels in the tail)": Impl(
        act={"gelu_erf": lambda x: 0.5 * x * (1 + sp.erf(x / math.sqrt(2)))}),
    "gelu_erf' drops x*phi": Impl(dact={"gelu_erf": sp.ndtr}),
    "gelu_erf' sign of x*phi flipped": Impl(dact={"gelu_erf": lambda x: sp.ndtr(x) - x * _phi(x)}),
    "gelu_tanh cubic typo 0.04715": Impl(
        act={"gelu_tanh": lambda x: x * _sig(2 * K * (x + 0.04715 * x ** 3))}),
    "gelu_tanh via 1+tanh (cancels in the tail)": Impl(
        act={"gelu_tanh": lambda x: 0.5 * x * (1 + np.tanh(K * (x + C3 * x ** 3)))}),
    "gelu_tanh' drops the 3 in 3*c*x^2": Impl(dact={"gelu_tanh": lambda x: (
        _sig(2 * K * (x + C3 * x ** 3))
        + 2 * x * K * (1 + C3 * x * x) * _sig(2 * K * (x + C3 * x ** 3)) * _sig(-2 * K * (x + C3 * x ** 3)))}),
    "gelu_tanh' drops the factor 2": Impl(dact={"gelu_tanh": lambda x: (
        _sig(2 * K * (x + C3 * x ** 3))
        + x * K * (1 + 3 * C3 * x * x) * _sig(2 * K * (x + C3 * x ** 3)) * _sig(-2 * K * (x + C3 * x ** 3)))}),
    "erf and tanh GELU swapped": Impl(act={"gelu_erf": lambda x: oracle.act("gelu_tanh", x),
                                           "gelu_tanh": lambda x: oracle.act("gelu_erf", x)},
                                      dact={"gelu_erf": lambda x: oracle.dact("gelu_tanh", x),
                                            "gelu_tanh": lambda x: oracle.dact("gelu_erf", x)}),
    "relu'(0) = 1": Impl(dact={"relu": lambda x: np.where(x >= 0, 1.0, 0.0)}),
    "relu drops NaN": Impl(act={"relu": lambda x: np.where(x > 0, x, 0.0)}),
    "da and db swapped": Impl(swap_grads=True),
    "activation applied to b": Impl(act_on_b=True),
    "db misses dy": Impl(drop_dy_db=True),
    "[gate | up] halves swapped": Impl(swap_halves=True),
}


def test_oracle_passes_every_pin():
    failures = pins.run_all(oracle)
    assert failures == [], "\n".join(failures)


def test_unmutated_assembly_passes():
    """The mutation harness itself is faithful when nothing is planted."""
    failures = pins.run_all(Impl())
    assert failures == [], "\n".join(failures)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    failures = pins.run_all(MUTANTS[name])
    assert failures, f"no pin caught: {name}"


def test_scalar_and_array_entry_points_agree():
    x = np.linspace(-9, 9, 37)
    for k in pins.KINDS:
        assert np.array_equal(oracle.act(k, x), [oracle.act1(k, v) for v in x])
        assert np.array_equal(oracle.dact(k, x), [oracle.dact1(k, v) for v in x])


def test_gate_up_split_shapes():
    x = np.arange(12.0).reshape(2, 6)
    a, b = oracle.split_gate_up(x)
    assert a.tolist() == [[0, 1, 2], [6, 7, 8]]
    assert b.tolist() == [[3, 4, 5], [9, 10, 11]]
    with pytest.raises(ValueError):
        oracle.split_gate_up(np.zeros((2, 5)))


def test_nan_propagates_every_kind():
    for k in pins.KINDS:
        assert np.isnan(oracle.act(k, [np.nan])[0])
        da, db = oracle.bwd(k, [np.nan], [1.0], [1.0])
        assert np.isnan(da[0]) and np.isnan(db[0])


def test_golden_oracle_points():
    """Regression guard: the oracle reproduces the values a committed script
    (tests/golden/make_oracle_points.py, which calls only the oracle) wrote.
    libm may differ by an ulp or two between hosts."""
    import os
    path = os.path.join(pins.GOLDEN, "oracle_points.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for kind, fn, x, v in rows:
        got = (oracle.act1 if fn == "act" else oracle.dact1)(kind, float.fromhex(x))
        want = float.fromhex(v)
        assert abs(got - want) <= 4 * 2.0 ** -52 * abs(want) + 1e-300, (kind, fn, x, got, want)
