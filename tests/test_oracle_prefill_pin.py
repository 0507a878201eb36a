"""Pin of the oracle's prefill (a6) expert FFN against a hand-worked case.

The composition the prefill reference follows -- x to MXFP6 along hidden,
gate/up, SwiGLU, h rounded to float32, h to MXFP6 along the expert width,
down -- is checked on the values of tests/golden/prefill_a6_hand.json, every
one of them worked out by hand.  Plausible mistakes in that composition are
then planted in the oracle (on the CPU, through monkeypatch) to show that the
hand values reject each of them.  CPU only.
"""
import json
import os

import numpy as np
import pytest

from gen import inputs as gi
from oracle import moe_oracle as o


def _case(golden_dir):
    with open(os.path.join(golden_dir, "prefill_a6_hand.json")) as f:
        g = json.load(f)
    H, I, T = g["shape"]["H"], g["shape"]["I"], g["shape"]["T"]

    def dense(entries, rows, cols):
        a = np.zeros((rows, cols))
        for r, c, v in entries:
            a[r, c] = v
        return a

    def matrix(spec, rows, K):
        codes = np.zeros((rows, K), np.uint8)
        for r, c, v in spec["codes"]:
            codes[r, c] = v
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)  # element 2c in the low nibble
        scales = np.full((rows, K // 32), g["default_scale_byte"], np.uint8)
        for r, b, v in spec["scales"]:
            scales[r, b] = v
        return packed, scales

    mats = {0: matrix(g["gate"], I, H), 1: matrix(g["up"], I, H), 2: matrix(g["down"], H, I)}
    x = dense(g["x"], T, H)
    return dict(g=g, H=H, I=I, T=T, mats=mats, x=x,
                x_bf16=gi.f32_to_bf16_bits(x.astype(np.float32)),
                q6_x=dense(g["q6_x"], T, H), g_=dense(g["g"], T, I), u=dense(g["u"], T, I),
                h=dense(g["h"], T, I), q6_h=dense(g["q6_h"], T, I), y=dense(g["y"], T, H))


def _run(c, mode="a6"):
    ids = np.zeros((c["T"], 1), np.int32)
    return o.ffn(c["x_bf16"], ids, lambda e, m: c["mats"][m], c["H"], mode)


def test_hand_case_inputs_are_exact(golden_dir):
    c = _case(golden_dir)
    assert np.array_equal(o.bf16_bits_to_f64(c["x_bf16"]), c["x"])  # every x is a bf16 value


def test_hand_case_intermediates(golden_dir):
    c = _case(golden_dir)
    wg = o.dequant(*c["mats"][0])
    wu = o.dequant(*c["mats"][1])
    q6x = o.q6_dequant(*o.q6_rows(c["x"]))
    assert np.array_equal(q6x, c["q6_x"])
    g = q6x @ wg.T
    u = q6x @ wu.T
    assert np.array_equal(g, c["g_"]) and np.array_equal(u, c["u"])
    h = o.swiglu(g, u)
    # h is g*u exactly wherever g >= 48; the one entry with g = -336 is about -3.5e-144
    pos = c["g_"] >= 48.0
    assert np.array_equal(h[pos], c["h"][pos])
    assert np.all(np.abs(h[~pos]) < 1e-140) and h[0, 6] < 0.0
    assert np.array_equal(o.q6_dequant(*o.q6_rows(o.round_f32(h))), c["q6_h"])


def test_hand_case_y(golden_dir):
    c = _case(golden_dir)
    y = _run(c)
    assert np.array_equal(y, c["y"])
    # the same rows through the whole layer (one expert, k = 1, weight 1): out = y
    out = o.combine(y, np.ones((c["T"], 1)))
    assert np.array_equal(out, c["y"])
    # the unquantised decode reference differs: the quantisation is visible in y
    assert not np.array_equal(_run(c, "a16"), c["y"])


def _plant(monkeypatch, call, procedure):
    """Plant a mistake in the oracle's quantisation step number `call` (0: x,
    1: h): that call returns procedure(values) instead of Q6(values), every
    other call stays as it is."""
    real_rows, real_deq = o.q6_rows, o.q6_dequant
    seen = {"n": 0}

    def rows(a):
        i = seen["n"]
        seen["n"] += 1
        a = np.asarray(a, np.float64)
        v = procedure(a, real_rows, real_deq) if i == call else real_deq(*real_rows(a))
        return ("planted", v), None

    def deq(codes, sb):
        return codes[1] if isinstance(codes, tuple) else real_deq(codes, sb)

    monkeypatch.setattr(o, "q6_rows", rows)
    monkeypatch.setattr(o, "q6_dequant", deq)


def _skip(a, rows, deq):
    return a


def _transposed(a, rows, deq):
    return deq(*rows(a.T)).T


_MISTAKES = {
    "x not quantised": (0, _skip),
    "h not quantised": (1, _skip),
    "x quantised along tokens instead of hidden": (0, _transposed),
    "h quantised along tokens instead of the expert width": (1, _transposed),
}


@pytest.mark.parametrize("mistake", list(_MISTAKES))
def test_planted_quantisation_mistakes_fail_the_hand_case(golden_dir, monkeypatch, mistake):
    """Each mistake, planted in the oracle, changes y on the hand case."""
    c = _case(golden_dir)
    _plant(monkeypatch, *_MISTAKES[mistake])
    assert not np.array_equal(_run(c), c["y"]), mistake


def test_planted_mistake_no_float32_rounding_of_h(golden_dir, monkeypatch):
    """Taking the quantisation decision of h on its fp64 value instead of the
    float32 value changes y[0][1] from 256 to 288 (the hand case's tie)."""
    c = _case(golden_dir)
    monkeypatch.setattr(o, "round_f32", lambda a: np.asarray(a, np.float64))
    y = _run(c)
    assert y[0, 1] == 288.0 and not np.array_equal(y, c["y"])


def test_planted_mistakes_leave_the_real_oracle_alone(golden_dir, monkeypatch):
    """The planting mechanism itself: a 'mistake' that quantises exactly as
    the oracle does reproduces the hand values."""
    c = _case(golden_dir)
    _plant(monkeypatch, 0, lambda a, rows, deq: deq(*rows(a)))
    assert np.array_equal(_run(c), c["y"])


def test_swiglu_before_quantisation_matters(golden_dir):
    """Quantising g and u instead of h gives a different y on the hand case."""
    c = _case(golden_dir)
    q6x = o.q6_dequant(*o.q6_rows(c["x"]))
    g = q6x @ o.dequant(*c["mats"][0]).T
    u = q6x @ o.dequant(*c["mats"][1]).T
    h = o.swiglu(o.q6_dequant(*o.q6_rows(g)), o.q6_dequant(*o.q6_rows(u)))
    y = h @ o.dequant(*c["mats"][2]).T
    assert not np.array_equal(y, c["y"])
