"""Pins of the oracle's router gate projection (router_logits, route_from_x)
against hand-worked values, exact rational arithmetic and closed forms."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from gen import inputs as gi
from oracle import moe_oracle as o


def bf16(a):
    return gi.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.fixture
def hand(golden_dir):
    with open(os.path.join(golden_dir, "router_gate_hand.json")) as f:
        return json.load(f)


def test_hand_logits(hand):
    x, w = bf16(hand["x"]), bf16(hand["w_router"])
    np.testing.assert_array_equal(o.router_logits(x, w), np.array(hand["logits_no_bias"]))
    np.testing.assert_array_equal(o.router_logits(x, w, np.array(hand["bias"], np.float32)),
                                  np.array(hand["logits_bias"]))
    # the transposed product x . W is a different matrix here: the pin sees it
    assert not np.array_equal(o.router_logits(x, w)[:1], np.array(hand["wrong_orientation_x_times_W"]))


def test_hand_routing(hand):
    x, w = bf16(hand["x"]), bf16(hand["w_router"])
    bias = np.array(hand["bias"], np.float32)
    for case in hand["route"]:
        _, ids, wt = o.route_from_x(x, w, case["k"], bias if case["bias"] else None)
        np.testing.assert_array_equal(ids, np.array(case["ids"]))
        np.testing.assert_allclose(wt.sum(axis=1), 1.0, rtol=0, atol=1e-15)
        if "w" in case:
            np.testing.assert_array_equal(wt, np.array(case["w"]))
    # closed forms of the k = 2 weights
    _, _, wt = o.route_from_x(x, w, 2, bias)
    assert wt[0, 0] == pytest.approx(1 / (1 + math.exp(-2)), abs=1e-15)
    assert wt[1, 1] == pytest.approx(math.exp(-13.25) / (1 + math.exp(-13.25)), abs=1e-15)
    _, _, wt = o.route_from_x(x, w, 2)
    assert wt[0, 1] == pytest.approx(math.exp(-3) / (1 + math.exp(-3)), abs=1e-15)


def test_exact_rational_brute_force():
    """Each logit against the exact rational dot product of the bf16 values:
    fp64 evaluation stays within H * 2^-53 * sum|x_c w_c| of it."""
    rng = np.random.default_rng(11)
    T, E, H = 3, 5, 64
    x = bf16(rng.standard_normal((T, H)))
    w = bf16(rng.standard_normal((E, H)) / 8)
    b = rng.standard_normal(E).astype(np.float32)
    got = o.router_logits(x, w, b)
    xv, wv = o.bf16_bits_to_f64(x), o.bf16_bits_to_f64(w)
    for t in range(T):
        for e in range(E):
            terms = [Fraction(float(xv[t, c])) * Fraction(float(wv[e, c])) for c in range(H)]
            exact = sum(terms, Fraction(0)) + Fraction(float(b[e]))
            bound = (H + 1) * 2.0 ** -53 * (float(sum(abs(q) for q in terms)) + abs(float(b[e])))
            assert abs(Fraction(float(got[t, e])) - exact) <= Fraction(bound)


def test_one_hot_rows_select_scaled_elements():
    """W_r[e] = 2^-s_e at column pi(e), zero elsewhere: logit = x[pi(e)] * 2^-s_e exactly."""
    rng = np.random.default_rng(5)
    T, E, H = 4, 12, 256
    x = bf16(rng.standard_normal((T, H)))
    pi = rng.permutation(H)[:E]
    s = rng.integers(0, 6, E)
    w = np.zeros((E, H), np.float32)
    w[np.arange(E), pi] = np.ldexp(1.0, -s)
    got = o.router_logits(x, bf16(w))
    want = o.bf16_bits_to_f64(x)[:, pi] * np.ldexp(1.0, -s)[None, :]
    np.testing.assert_array_equal(got, want)


def test_zero_gate_routes_by_bias():
    """W_r = 0: the logits are the bias and the top-k are the largest biases."""
    rng = np.random.default_rng(9)
    T, E, H, k = 3, 16, 32, 4
    b = rng.permutation(E).astype(np.float32) - 7.5
    l, ids, _ = o.route_from_x(bf16(rng.standard_normal((T, H))), np.zeros((E, H), np.uint16), k, b)
    np.testing.assert_array_equal(l, np.broadcast_to(b.astype(np.float64), (T, E)))
    want = np.argsort(-b, kind="stable")[:k]
    np.testing.assert_array_equal(ids, np.broadcast_to(want, (T, k)))


def test_masked_routing_and_linearity():
    """Masked experts never appear; scaling x by 2 scales the bias-free logits by 2 exactly."""
    rng = np.random.default_rng(3)
    T, E, H, k = 5, 10, 64, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = bf16(rng.standard_normal((E, H)) / 8)
    l1 = o.router_logits(bf16(x), w)
    l2 = o.router_logits(bf16(2 * x), w)
    np.testing.assert_array_equal(l2, 2 * l1)
    e2s = np.array([0, -1, 1, -1, 2, 3, -1, 4, 5, 6], np.int32)
    _, ids, _ = o.route_from_x(bf16(x), w, k, None, e2s)
    assert np.all(e2s[ids] >= 0)


def test_router_weight_statistics():
    """The synthetic W_r gives logits of about unit variance on x ~ N(0,1)."""
    cfg = gi.custom("r", 1024, 128, 64, 8, 32)
    hi = gi.host_inputs(cfg)
    l = o.router_logits(hi.x_bf16, gi.router_weights(cfg))
    assert 0.8 < float(np.std(l)) < 1.2
