"""Pins of the oracle's cb3 codec (cb3_indices, cb3_dequant, ffn_cb3) against
hand-worked bytes, brute-force bit extraction and an integer-exact FFN."""
import json
import os

import numpy as np

from gen import inputs as gi
from oracle import moe_oracle as o


def bf16(a):
    return gi.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_hand_unpack_and_dequant(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cb3_hand.json")))
    for case in g["unpack"]:
        got = o.cb3_indices(np.array([case["bytes"]], np.uint8), 8)
        np.testing.assert_array_equal(got[0], case["indices"])
    d = g["dequant"]
    w = o.cb3_dequant(np.array(d["bytes"], np.uint8), bf16(d["codebook"]))
    np.testing.assert_array_equal(w, np.array(d["weights"]))


def test_unpack_against_bitwise_brute_force():
    """Every index against a bit-by-bit read of the row's little-endian bit stream."""
    rng = np.random.default_rng(4)
    rows, K = 3, 64
    q = rng.integers(0, 256, (rows, K * 3 // 8), dtype=np.uint8)
    got = o.cb3_indices(q, K)
    for r in range(rows):
        bits = [(int(q[r, i // 8]) >> (i % 8)) & 1 for i in range(K * 3)]
        for c in range(K):
            assert got[r, c] == bits[3 * c] | (bits[3 * c + 1] << 1) | (bits[3 * c + 2] << 2)


def test_ffn_cb3_integer_exact():
    """H = I = 32, one expert: gate rows all 1 (g = 64), up rows all 0.5
    (u = 32, h = silu(64) * 32), down rows all 1.5: y = 32 * 1.5 * h."""
    H = I = 32
    x = bf16(np.full((1, H), 2.0))
    ones = np.zeros((I, H * 3 // 8), np.uint8)          # index 0 everywhere
    def cb(v, rows):
        c = np.zeros((rows, 8), np.float32)
        c[:, 0] = v
        return bf16(c)
    mats = {0: (ones, cb(1.0, I)), 1: (ones, cb(0.5, I)), 2: (np.zeros((H, I * 3 // 8), np.uint8), cb(1.5, H))}
    y = o.ffn_cb3(x, np.array([[0]], np.int32), lambda e, m: mats[m], H)
    h = 64.0 * 32.0 / (1.0 + np.exp(-64.0))
    np.testing.assert_allclose(y, np.full((1, H), 32 * 1.5 * h), rtol=1e-15)
    assert h == 2048.0   # silu(64) == 64 in fp64


def test_ffn_cb3_matches_dense_definition_and_generator():
    """ffn_cb3 equals the plain FFN on explicitly decoded matrices; the host
    generator gives codebooks of the stated statistics and uniform indices."""
    cfg = gi.custom("cb3", 256, 128, 4, 2, 3, seed=41)
    hi = gi.host_inputs(cfg)
    w = gi.HostCb3Weights(cfg)
    ids = np.array([[0, 3], [1, 0], [2, 3]], np.int32)
    y = o.ffn_cb3(hi.x_bf16, ids, w.matrix, cfg.H)
    x = o.bf16_bits_to_f64(hi.x_bf16)
    for p in range(6):
        e = int(ids.reshape(-1)[p])
        g = o.cb3_dequant(*w.matrix(e, 0)) @ x[p // 2]
        u = o.cb3_dequant(*w.matrix(e, 1)) @ x[p // 2]
        ref = o.cb3_dequant(*w.matrix(e, 2)) @ (g * u / (1 + np.exp(-g)))
        np.testing.assert_allclose(y[p], ref, rtol=1e-12, atol=1e-12)
    idx = o.cb3_indices(*w.matrix(0, 0)[:1], cfg.H)
    counts = np.bincount(idx.reshape(-1), minlength=8)
    assert counts.min() > 0.8 * idx.size / 8
    cb = o.bf16_bits_to_f64(w.matrix(0, 2)[1])
    assert 0.09 < float(np.std(cb)) < 0.16
