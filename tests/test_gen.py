"""Input generator checks (CPU): SplitMix64 known answers and the value
distributions the synthetic workloads promise."""
import numpy as np

from gen import inputs as gi
from gen import splitmix as sm


def test_splitmix64_known_answers():
    # SplitMix64 state 1234567: the first five outputs of the published generator
    assert [int(v) for v in sm.outputs(1234567, 0, 5)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]
    assert sm.mix64_int(0) == 0


def test_counter_access_is_random_access():
    s0 = sm.stream_seed(1002, 0, 17, sm.MATRIX_UP, sm.KIND_CODES)
    full = sm.outputs(s0, 0, 1000)
    np.testing.assert_array_equal(sm.outputs(s0, 400, 100), full[400:500])


def test_code_and_scale_distributions():
    b = sm.code_bytes(1002, 0, 3, sm.MATRIX_GATE, 1 << 20)
    lo, hi = np.bincount(b & 15, minlength=16), np.bincount(b >> 4, minlength=16)
    exp = len(b) / 16
    assert np.all(np.abs(lo - exp) < 6 * np.sqrt(exp)) and np.all(np.abs(hi - exp) < 6 * np.sqrt(exp))
    for emin in (-4, -6):
        s = sm.scale_bytes(1002, 0, 3, sm.MATRIX_DOWN, 70000, emin)
        assert s.min() == 127 + emin and s.max() == 127
        c = np.bincount(s - (127 + emin))
        assert len(c) == 1 - emin and np.all(np.abs(c - 70000 / (1 - emin)) < 6 * np.sqrt(70000 / (1 - emin)))


def test_streams_differ_by_key():
    a = sm.code_bytes(1002, 0, 3, 0, 64)
    assert not np.array_equal(a, sm.code_bytes(1002, 0, 4, 0, 64))
    assert not np.array_equal(a, sm.code_bytes(1002, 1, 3, 0, 64))
    assert not np.array_equal(a, sm.code_bytes(1002, 0, 3, 1, 64))
    assert not np.array_equal(a, sm.code_bytes(1003, 0, 3, 0, 64))


def test_host_inputs_shapes_and_determinism():
    for name in ("tiny", "verify16"):
        cfg = gi.CONFIGS[name]
        a, b = gi.host_inputs(cfg), gi.host_inputs(cfg)
        assert a.x_bf16.shape == (cfg.T, cfg.H) and a.x_bf16.dtype == np.uint16
        assert a.logits[0].shape == (cfg.T, cfg.E) and a.logits[0].dtype == np.float32
        np.testing.assert_array_equal(a.x_bf16, b.x_bf16)
        np.testing.assert_array_equal(a.logits[0], b.logits[0])
    cfg = gi.CONFIGS["chain40"]
    # only the resident subsets and small arrays are materialised here
    hi = gi.host_inputs(cfg)
    assert len(hi.resident) == 40 and all(len(r) == 154 for r in hi.resident)
    assert all(np.all(np.diff(r) > 0) for r in hi.resident)
    for r, t in zip(hi.resident, hi.expert_to_slot):
        assert np.all(t[r] == np.arange(154)) and np.count_nonzero(t >= 0) == 154


def test_zipf_bias_skews_routing():
    cfg = gi.CONFIGS["verify16"]
    hi = gi.host_inputs(cfg)
    ranks = np.exp(-hi.bias / cfg.zipf)
    assert sorted(np.round(ranks).astype(int).tolist()) == list(range(1, cfg.E + 1))


def test_bf16_input_rounding_matches_torch():
    import torch
    a = np.random.default_rng(0).standard_normal(4096).astype(np.float32)
    ours = gi.f32_to_bf16_bits(a)
    theirs = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
