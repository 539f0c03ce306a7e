"""CPU pins of the Floyd attention oracle (oracle/floyd.py; page "CANN
Floyd注意力梯度算子", sections 功能说明 and 调用示例), and planted mistakes that
at least one pin must reject.  The mistakes are planted in a private copy of
the oracle's source on the CPU."""

import os
import types

import numpy as np
import pytest

from floyd_pins import PINS, rand_problem

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "floyd.py")

MUTATIONS = {
    "dq_drops_k2_term": ("dq = scale * (ds @ k1 + _from_m(_by_m(ds) @ _by_m(k2)))", "dq = scale * (ds @ k1)"),
    "dq_k1_batched_over_m": ("dq = scale * (ds @ k1 + _from_m(_by_m(ds) @ _by_m(k2)))",
                             "dq = scale * (_from_m(_by_m(ds) @ _by_m(k2)) + _from_m(_by_m(ds) @ _by_m(k2)))"),
    "dp_drops_v2_term": ("dp = dy @ _swap(v1) + _from_m(_by_m(dy) @ _swap(_by_m(v2)))", "dp = dy @ _swap(v1)"),
    "dropped_sfmg": ("ds = p * (dp - sfmg[..., None])", "ds = p * dp"),
    "sign_flip_ds": ("ds = p * (dp - sfmg[..., None])", "ds = p * (sfmg[..., None] - dp)"),
    "dk2_uses_p": ("dk2 = scale * _from_m(_swap(_by_m(ds)) @ _by_m(q))",
                   "dk2 = scale * _from_m(_swap(_by_m(p)) @ _by_m(q))"),
    "dv2_uses_ds": ("dv2 = _from_m(_swap(_by_m(p)) @ _by_m(dy))", "dv2 = _from_m(_swap(_by_m(ds)) @ _by_m(dy))"),
    "dk1_without_scale": ("dk1 = scale * (_swap(ds) @ q)", "dk1 = _swap(ds) @ q"),
    "scale_on_k1_only": ("s = scale * (t1 + t2)", "s = scale * t1 + t2"),
    "mask_inverted": ("s = np.where(mb, -np.inf, s)", "s = np.where(~mb, -np.inf, s)"),
    "p_not_normalised": ("p = np.exp(s - safe_mx[..., None]) / safe_sm[..., None]",
                         "p = np.exp(s - safe_mx[..., None])"),
    "y_drops_v2_term": ("y = p @ v1 + _from_m(_by_m(p) @ _by_m(v2))", "y = p @ v1"),
    "stats_last_copy_wrong": ("sm = np.asarray(softmax_sum, dtype=np.float64)[..., 0]",
                              "sm = np.asarray(softmax_sum, dtype=np.float64)[..., 0] * 1.0001"),
}


def load(name=None):
    src = open(SRC, encoding="utf-8").read()
    if name is not None:
        old, new = MUTATIONS[name]
        assert src.count(old) == 1, f"mutation anchor missing: {name}"
        src = src.replace(old, new)
    mod = types.ModuleType(f"floyd_{name or 'plain'}")
    exec(compile(src, f"<floyd {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("pin", sorted(PINS))
def test_oracle_passes_pin(pin):
    import oracle.floyd as F

    assert not PINS[pin](F), pin


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = load(name)
    caught = [p for p, f in PINS.items() if f(mod)]
    assert caught, f"no pin rejects {name}"


def test_fully_masked_row_gives_zeros():
    import oracle.floyd as F

    q, k1, v1, k2, v2, dy, mask = rand_problem(1, 1, 2, 3, 4, 2, 5, ((0, 0),), 0.0)
    y, mx, sm = F.forward(q, k1, v1, k2, v2, 0.5, mask)
    assert np.all(mx[0, 0, 0] == -np.inf) and np.all(sm[0, 0, 0] == 0) and not np.any(y[0, 0, 0])
    g = F.backward(q, k1, v1, k2, v2, dy, y, mx, sm, 0.5, mask)
    assert not np.any(g[0][0, 0, 0]) and not np.any(g[1][0, 0, 0]) and not np.any(g[2][0, 0, 0])


def test_flop_count():
    import oracle.floyd as F

    mask = np.zeros((2, 1, 4, 1, 8), dtype=bool)
    mask[0, 0, 1, 0, :3] = True
    assert F.flops(2, 3, 4, 5, 8, 16) == 20 * 16 * 2 * 3 * 4 * 5 * 8
    assert F.flops(2, 3, 4, 5, 8, 16, mask) == 20 * 16 * 3 * 5 * (2 * 4 * 8 - 3)
