"""Pins of the CPU oracle against hand-worked values, closed forms and
invariants that do not come from the oracle itself.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from gen import inputs as gi


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats

def test_e2m1_table_matches_hand_values(golden_dir):
    g = load(golden_dir, "e2m1_ue8m0_hand.json")
    tab = o.E2M1_TABLE
    assert list(tab) == g["e2m1_table"]
    assert all(math.copysign(1, a) == math.copysign(1, b) for a, b in zip(tab, g["e2m1_table"]))
    assert tab.sum() == 0.0
    assert sorted(set(abs(v) for v in tab)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_packed_bytes_and_nibble_order(golden_dir):
    g = load(golden_dir, "e2m1_ue8m0_hand.json")
    for case in g["bytes"]:
        v = o.decode_codes(np.array([[case["byte"]]], dtype=np.uint8))[0]
        assert list(v) == case["elements"], case
        assert [math.copysign(1, a) for a in v] == [math.copysign(1, b) for b in case["elements"]]


def test_ue8m0(golden_dir):
    g = load(golden_dir, "e2m1_ue8m0_hand.json")
    for case in g["scales"]:
        assert o.ue8m0_value(case["byte"]) == case["value"]
    with pytest.raises(ValueError):
        o.ue8m0_value(255)
    with pytest.raises(ValueError):
        o.dequant(np.zeros((1, 16), np.uint8), np.full((1, 1), 255, np.uint8))


def test_weighted_examples(golden_dir):
    g = {c["what"]: c["value"] for c in load(golden_dir, "e2m1_ue8m0_hand.json")["weighted"]}
    # code 7 at scale 121: a single element row padded with zero codes
    codes = np.zeros((1, 16), np.uint8)
    codes[0, 0] = 0x07
    w = o.dequant(codes, np.array([[121]], np.uint8))
    assert w[0, 0] == g["code 7 (6.0) with scale byte 121"]
    w = o.dequant(np.full((1, 16), 0x22, np.uint8), np.array([[126]], np.uint8))
    assert w.sum() == g["row of 32 codes 1.0 (bytes 0x22), scale byte 126, dot with x = 1"]
    w = o.dequant(np.full((1, 16), 0xF7, np.uint8), np.array([[127]], np.uint8))
    assert w.sum() == g["row of 16 bytes 0xF7, scale byte 127, dot with x = 1"]


def test_scale_block_boundaries():
    # one row of K=96: three blocks with scales 2^-1, 2^0, 2^3, all codes 1.0
    codes = np.full((1, 48), 0x22, np.uint8)
    w = o.dequant(codes, np.array([[126, 127, 130]], np.uint8))[0]
    assert np.all(w[:32] == 0.5) and np.all(w[32:64] == 1.0) and np.all(w[64:] == 8.0)


# ---------------------------------------------------------------- byte model

def test_byte_model_matches_pages(golden_dir):
    g = load(golden_dir, "byte_model.json")
    cfg = gi.CONFIGS["decode1"]
    assert cfg.H == g["hidden"] and cfg.I == g["expert_width"] and cfg.E == g["experts_per_layer"]
    assert g["layers"] * g["experts_per_layer"] == g["routed_experts"]
    assert cfg.expert_bytes == 18_800_640
    assert round(cfg.expert_bytes / 1e6, 1) == g["expert_MB"]
    weights = g["routed_experts"] * 3 * cfg.H * cfg.I
    assert round(weights / 1e9, 1) == g["routed_weights_billion"]
    assert round(g["routed_experts"] * cfg.expert_bytes / 1e9, 1) == g["routed_bytes_GB"]
    assert round(g["arena_slots"] * cfg.expert_bytes / 1e9, 1) == g["arena_GB"]
    assert round(100 * g["arena_slots"] / g["routed_experts"], 1) == g["arena_fraction_percent"]
    chain = gi.CONFIGS["chain40"]
    assert chain.layers * chain.resident * chain.expert_bytes == 115_811_942_400


# ---------------------------------------------------------------- router

def test_route_hand_cases(golden_dir):
    g = load(golden_dir, "route_permute_hand.json")
    for case in g["route"]:
        logits = np.array(case["logits"], dtype=np.float32)
        e2s = np.array(case["expert_to_slot"], np.int32) if "expert_to_slot" in case else None
        ids, w = o.route(logits, case["k"], e2s)
        assert ids.tolist() == case["ids"]
        if "w" in case:
            np.testing.assert_allclose(w, case["w"], rtol=0, atol=1e-7)
    # exact closed form for the masked case: logits 4 and 3 selected
    ids, w = o.route(np.array([[5, 1, 4, 3]], np.float32), 2, np.array([-1, 0, 1, 2], np.int32))
    assert w[0, 0] == pytest.approx(1 / (1 + math.exp(-1)), abs=1e-15)
    # k = 1 gives exactly one
    _, w = o.route(np.array([[0.3, -2.0]], np.float32), 1)
    assert w[0, 0] == 1.0


def test_route_ln3_closed_form():
    l0 = np.float32(math.log(3.0))
    _, w = o.route(np.array([[l0, 0.0, -5.0]], np.float32), 2)
    e = math.exp(float(l0))
    assert w[0, 0] == pytest.approx(e / (e + 1), abs=1e-15)
    assert abs(w[0, 0] - 0.75) < 1e-7


def test_route_invariants_random():
    rng = np.random.default_rng(5)
    for T, E, k in [(7, 8, 2), (5, 33, 8), (3, 384, 8), (2, 16, 16)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        logits[0, :4] = logits[0, 4]                        # force ties
        e2s = np.where(rng.random(E) < 0.7, 0, -1).astype(np.int32)
        e2s[:k] = 0
        ids, w = o.route(logits, k, e2s)
        assert np.all(np.abs(w.sum(1) - 1) < 1e-14)
        for t in range(T):
            chosen = set(ids[t].tolist())
            assert len(chosen) == k and all(e2s[e] >= 0 for e in chosen)
            # every chosen expert beats every unchosen routable expert under (logit desc, index asc)
            for a in chosen:
                for b in range(E):
                    if b in chosen or e2s[b] < 0:
                        continue
                    assert (logits[t, a] > logits[t, b]) or (logits[t, a] == logits[t, b] and a < b)
            # slots in rank order; weights non-increasing
            assert all(w[t, j] >= w[t, j + 1] for j in range(k - 1))
            for j in range(k - 1):
                a, b = ids[t, j], ids[t, j + 1]
                assert (logits[t, a] > logits[t, b]) or (logits[t, a] == logits[t, b] and a < b)


def test_route_rejects():
    with pytest.raises(ValueError):
        o.route(np.array([[np.nan, 0.0]], np.float32), 1)
    with pytest.raises(ValueError):
        o.route(np.array([[1.0, 0.0]], np.float32), 3)
    with pytest.raises(ValueError):
        o.route(np.array([[1.0, 0.0]], np.float32), 0)


def test_route_fewer_routable_than_k(golden_dir):
    """R-ROUTE-FILL hand cases, and the rows of the filled slots are zero."""
    for case in load(golden_dir, "route_permute_hand.json")["route_fill"]["cases"]:
        e2s = np.array(case["expert_to_slot"], np.int32)
        ids, w = o.route(np.array(case["logits"], np.float32), case["k"], e2s)
        assert ids.tolist() == case["ids"], case
        if "w" in case:
            assert w.tolist() == case["w"], case
    _, w = o.route(np.array([[3.0, 1.0, 4.0, 0.0, 2.0]], np.float32), 4, np.array([0, -1, -1, 1, -1], np.int32))
    e = math.exp(-3.0)
    assert w[0, 0] == pytest.approx(1 / (1 + e), abs=1e-15) and w[0, 1] == pytest.approx(e / (1 + e), abs=1e-15)
    assert w[0, 2] == 0.0 and w[0, 3] == 0.0
    # the FFN rows of an expert without a slot are zero; the routable rows are untouched
    H = I = 32
    mats = {0: (np.full((I, H // 2), 0x22, np.uint8), np.full((I, 1), 127, np.uint8)),
            1: (np.full((I, H // 2), 0x11, np.uint8), np.full((I, 1), 127, np.uint8)),
            2: (np.full((H, I // 2), 0x33, np.uint8), np.full((H, 1), 125, np.uint8))}
    x = _bf16(np.full((1, H), 2.0))
    e2s = np.array([0, -1], np.int32)
    y = o.ffn(x, np.array([[0, 1]], np.int32), lambda e, m: mats[m], H, "a16", e2s)
    assert np.all(y[0] == 24576.0) and np.all(y[1] == 0.0)


# ---------------------------------------------------------------- permutation

def test_permute_hand_cases(golden_dir):
    for case in load(golden_dir, "route_permute_hand.json")["permute"]:
        off, sp, p2r = o.permute(np.array(case["ids"], np.int32), case["E"])
        assert off.tolist() == case["offsets"]
        assert sp.tolist() == case["sorted_pair"]
        assert p2r.tolist() == case["pair_to_row"]


def test_permute_invariants_random():
    rng = np.random.default_rng(9)
    for T, E, k in [(1, 384, 8), (16, 384, 8), (100, 7, 3)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        off, sp, p2r = o.permute(ids, E)
        flat = ids.reshape(-1)
        assert sorted(sp.tolist()) == list(range(T * k))
        assert np.all(p2r[sp] == np.arange(T * k))
        for e in range(E):
            seg = sp[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
            assert off[e + 1] - off[e] == np.count_nonzero(flat == e)


# ---------------------------------------------------------------- FFN

def _weights_from(mats):
    return lambda e, m: mats[m]


def _bf16(vals):
    return gi.f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_ffn_integer_exact_case():
    # H = I = 32, x = 2; gate all 1.0 (scale 1), up all 0.5 (scale 1), down 1.5 at scale 0.25
    H = I = 32
    mats = {
        0: (np.full((I, H // 2), 0x22, np.uint8), np.full((I, 1), 127, np.uint8)),
        1: (np.full((I, H // 2), 0x11, np.uint8), np.full((I, 1), 127, np.uint8)),
        2: (np.full((H, I // 2), 0x33, np.uint8), np.full((H, 1), 125, np.uint8)),
    }
    x = _bf16(np.full((1, H), 2.0))
    y = o.ffn(x, np.array([[0]], np.int32), _weights_from(mats), H)
    # g = 64, silu(64) = 64 in fp64, u = 32, h = 2048, y = 32 * 0.375 * 2048
    assert np.all(y == 24576.0)
    out = o.combine(y, np.array([[1.0]]))
    assert np.all(out == 24576.0)


def test_ffn_structured_orientation_case():
    # H = 64, I = 32.  x has a single 1 at c = 5 (high nibble of byte 2).
    # gate row 3 has code 2.0 at c = 5, block 0 scale 2^1 -> g_3 = 4, other rows 0.
    # up: every row has 1.0 at c = 5 -> u = 1.  h = silu(g) -> only h_3 = silu(4) != 0.
    # down row 10 has 1.0 at n = 3 -> y_10 = silu(4); every other output 0.
    H, I = 64, 32
    gc = np.zeros((I, H // 2), np.uint8)
    gc[3, 2] = 0x40                      # element 5 = high nibble of byte 2 = code 4 (2.0)
    gs = np.full((I, H // 32), 127, np.uint8)
    gs[3, 0] = 128                       # block 0 of row 3 scaled by 2
    gs[3, 1] = 120                       # block 1 differs, must not be used for c = 5
    uc = np.zeros((I, H // 2), np.uint8)
    uc[:, 2] = 0x20                      # code 2 (1.0) at element 5
    us = np.full((I, H // 32), 127, np.uint8)
    dc = np.zeros((H, I // 2), np.uint8)
    dc[10, 1] = 0x20                     # element 3 = high nibble of byte 1 -> 1.0
    ds = np.full((H, I // 32), 127, np.uint8)
    mats = {0: (gc, gs), 1: (uc, us), 2: (dc, ds)}
    xv = np.zeros((1, H), np.float32)
    xv[0, 5] = 1.0
    y = o.ffn(_bf16(xv), np.array([[0]], np.int32), _weights_from(mats), H)
    expect = np.zeros(H)
    expect[10] = 4.0 / (1.0 + math.exp(-4.0))
    np.testing.assert_array_equal(y[0], expect)
    # gate and up play different roles: swap them and the result changes
    y2 = o.ffn(_bf16(xv), np.array([[0]], np.int32), _weights_from({0: (uc, us), 1: (gc, gs), 2: (dc, ds)}), H)
    assert y2[0, 10] == pytest.approx(4.0 * 1.0 / (1.0 + math.exp(-1.0)))
    assert y2[0, 10] != y[0, 10]


def test_ffn_scale_and_sign_invariants():
    cfg = gi.custom("inv", 64, 32, 4, 2, 3, emin=-3, seed=11)
    hi = gi.host_inputs(cfg)
    hw = gi.HostWeights(cfg)
    ids, _ = o.route(hi.logits[0], cfg.k)
    base = o.ffn(hi.x_bf16, ids, hw.matrix, cfg.H)

    def mod(fn):
        return lambda e, m: fn(m, *hw.matrix(e, m))

    # all down scales +1 -> y doubles exactly
    y = o.ffn(hi.x_bf16, ids, mod(lambda m, c, s: (c, s + (m == 2))), cfg.H)
    np.testing.assert_array_equal(y, 2 * base)
    # negate every up code (flip both sign bits) -> u, h and y negate exactly
    y = o.ffn(hi.x_bf16, ids, mod(lambda m, c, s: (c ^ (0x88 if m == 1 else 0), s)), cfg.H)
    np.testing.assert_array_equal(y, -base)
    # per-pair evaluation equals the bucketed evaluation (expert order does not matter)
    x = o.bf16_bits_to_f64(hi.x_bf16)
    for p in range(cfg.T * cfg.k):
        t, j = divmod(p, cfg.k)
        yp = o.expert_ffn(x[t:t + 1], hw.matrix, int(ids[t, j]))
        np.testing.assert_allclose(yp[0], base[p], rtol=1e-13, atol=0)


def test_combine_closed_form():
    y = np.array([[4.0, -1.0], [8.0, 3.0]])
    w = np.array([[0.75, 0.25]])
    out = o.combine(y, w)
    np.testing.assert_array_equal(out, [[5.0, 0.0]])
    res = _bf16([[1.5, -2.0]])
    np.testing.assert_array_equal(o.combine(y, w, res), [[6.5, -2.0]])


# ---------------------------------------------------------------- quantiser and bf16

def test_e2m3_table():
    tab = o.E2M3_TABLE
    assert tab.sum() == 0.0
    mags = sorted(set(abs(v) for v in tab))
    assert mags == [i / 8 for i in range(8)] + [1 + i / 8 for i in range(8)] + \
        [2 + i / 4 for i in range(8)] + [4 + i / 2 for i in range(8)]
    assert tab.max() == 7.5 and tab[0x1F] == 7.5 and tab[0x3F] == -7.5


def test_q6_hand_cases(golden_dir):
    for case in load(golden_dir, "q6_hand.json")["cases"]:
        v = np.zeros(32)
        v[:len(case["elements"])] = case["elements"]
        codes, sb = o.q6_block(v)
        assert sb == case["scale_byte"], case
        assert codes[:len(case["codes"])].tolist() == case["codes"], case
        assert np.all(codes[len(case["codes"]):] == 0)


def _brute_e2m3(t):
    """Nearest e2m3 code by exhaustive search over the 32 magnitudes; ties to the even code."""
    mags = o.E2M3_TABLE[:32]
    a = np.abs(t)[..., None]
    d = np.abs(mags[None, :] - a)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(32), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))
    code = np.where(np.abs(t) > 7.5, 31, code)
    return (code | np.where(np.signbit(t), 0x20, 0)).astype(np.uint8)


def test_e2m3_rounding_against_brute_force():
    rng = np.random.default_rng(6)
    t = np.concatenate([rng.uniform(-7.5, 7.5, 20000), np.arange(-60, 61) / 8.0, np.arange(-60, 61) / 16.0,
                        np.arange(8, 16) / 2 + 0.25, [0.0, -0.0, 1e-9, -1e-9]])
    np.testing.assert_array_equal(o.e2m3_encode(t), _brute_e2m3(t))


def test_q6_scale_is_smallest_non_saturating():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal((200, 64)) * np.exp(rng.uniform(-20, 20, (200, 1)))).astype(np.float32)
    a = a.astype(np.float64)
    codes, sb = o.q6_rows(a)
    amax = np.abs(a.reshape(200, 2, 32)).max(-1)
    X = sb.astype(np.int64) - 127
    # brute force: the smallest integer X with amax * 2^-X <= 7.5
    for i in range(200):
        for b in range(2):
            x = -140
            while np.ldexp(amax[i, b], -x) > 7.5:
                x += 1
            assert X[i, b] == x
    # and the codes are the nearest grid points of v * 2^-X
    t = np.ldexp(a.reshape(200, 2, 32), -X[..., None]).reshape(200, 64)
    np.testing.assert_array_equal(codes, _brute_e2m3(t))


def test_q6_exhaustive_bf16_against_brute_force():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    vals = vals[np.isfinite(vals)]
    vals = vals[: len(vals) // 32 * 32].reshape(-1, 32)
    codes, sb = o.q6_rows(vals)
    X = sb.astype(np.int64) - 127
    t = np.ldexp(vals.reshape(-1, 1, 32), -X[..., None]).reshape(vals.shape)
    zero_blocks = np.max(np.abs(vals), axis=1) == 0
    np.testing.assert_array_equal(codes[~zero_blocks], _brute_e2m3(t[~zero_blocks]))
    assert np.all(codes[zero_blocks] == 0) and np.all(sb[zero_blocks] == 0)


def test_q6_dequant_error_bound():
    # every element is within half a step of its grid: 2^-4 relative in the normal
    # binades, 1/16 absolute (times the block scale) below 1
    rng = np.random.default_rng(8)
    a = rng.standard_normal((64, 256))
    codes, sb = o.q6_rows(a)
    back = o.q6_dequant(codes, sb)
    scale = np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=1)
    t = np.abs(a) / scale
    bound = np.where(t >= 1, np.ldexp(1.0, np.frexp(t)[1] - 1 - 4), 1 / 16) * scale
    assert np.all(np.abs(back - a) <= bound * (1 + 1e-12))


def test_bf16_rne_against_torch():
    rng = np.random.default_rng(4)
    a = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-30, 30, 10000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 0.0, 2.0 ** -130, 3e38]])
    a32 = a.astype(np.float32)            # values exactly representable in float32
    ours = o.bf16_rne(a32.astype(np.float64))
    theirs = torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    assert o.bf16_rne(np.array([1 + 2 ** -8]))[0] == 0x3F80
    assert o.bf16_rne(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82


def test_bf16_rne_from_fp64_is_single_rounding():
    # 1 + 2^-8 + 2^-40 lies just above the bf16 midpoint: a direct fp64 rounding goes up,
    # while rounding through float32 first would land on the midpoint and go to even (down).
    v = 1 + 2 ** -8 + 2 ** -40
    assert o.bf16_rne(np.array([v]))[0] == 0x3F81


def test_rmsnorm_closed_form():
    x = _bf16(np.full((1, 64), 2.0))
    n = o.rmsnorm_bf16(x)
    assert np.all(n == 0x3F80)                       # 2/sqrt(4+1e-6) rounds to 1.0
    xv = np.tile([3.0, -4.0], 32)[None]
    n = o.bf16_bits_to_f64(o.rmsnorm_bf16(_bf16(xv)))
    r = math.sqrt(12.5 + 1e-6)
    np.testing.assert_allclose(n[0, :2], [3 / r, -4 / r], rtol=2 ** -8)
