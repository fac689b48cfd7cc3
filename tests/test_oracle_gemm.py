"""CPU tests of the oracle's gate/up projection with the fused activation:
its pins, and planted mistakes (in numpy copies built here) that each pin
set must catch."""
import numpy as np
import pytest

import oracle
import pins_gemm as pins


class Impl:
    def __init__(self, fn):
        self.gemm_glu = fn


def _mk(swap=False, act_on_up=False, no_act=False, drop_last_k=False, w_in_out=False, neg=False,
        x_transposed=False, u_from_gate=False):
    def fn(kind, x, wg, wu, want_gu=False):
        x, wg, wu = (np.asarray(v, np.float64) for v in (x, wg, wu))
        if w_in_out:      # weights read as [in][out] from the same memory
            wg = wg.reshape(wg.shape[1], wg.shape[0]).T
            wu = wu.reshape(wu.shape[1], wu.shape[0]).T
        if x_transposed:  # x read as [k][m] from the same memory
            x = x.reshape(x.shape[1], x.shape[0]).T
        if drop_last_k:
            x, wg, wu = x[:, :-1], wg[:, :-1], wu[:, :-1]
        g, u = x @ wg.T, x @ wu.T
        if u_from_gate:
            u = g.copy()
        if neg:
            g = -g
        if swap:
            g, u = u, g
        if no_act:
            h = g * u
        elif act_on_up:
            h = g * pins.torch_act(kind, u)
        else:
            h = pins.torch_act(kind, g) * u
        return (h, g, u) if want_gu else h
    return Impl(fn)


MUTANTS = {
    "gate and up swapped": _mk(swap=True),
    "activation on the up projection": _mk(act_on_up=True),
    "activation missing": _mk(no_act=True),
    "last k term dropped": _mk(drop_last_k=True),
    "weights read as [in][out]": _mk(w_in_out=True),
    "gate sign flipped": _mk(neg=True),
    "x transposed": _mk(x_transposed=True),
    "up computed from the gate weights": _mk(u_from_gate=True),
}


def test_oracle_passes_gemm_pins():
    f = pins.run_all(oracle)
    assert f == [], "\n".join(f)


def test_faithful_copy_passes():
    f = pins.run_all(_mk())
    assert f == [], "\n".join(f)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gemm_pins_catch_planted_mistake(name):
    assert pins.run_all(MUTANTS[name]), f"no pin caught: {name}"


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.gemm_glu("silu", np.zeros((2, 3)), np.zeros((4, 3)), np.zeros((4, 2)))
    with pytest.raises(ValueError):
        oracle.gemm_glu("silu", np.zeros((2, 3)), np.zeros((4, 5)), np.zeros((4, 5)))
