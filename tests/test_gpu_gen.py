"""The device filler reproduces the host SplitMix64 streams byte for byte."""
import numpy as np
import pytest

from gen import device as gd
from gen import inputs as gi
from gen import splitmix as sm

pytestmark = pytest.mark.gpu


def test_device_fill_matches_host_streams():
    cfg = gi.custom("fillcheck", 512, 256, 16, 2, 1, emin=-6, seed=4242)
    slot_expert = np.array([5, 0, 15, 9], dtype=np.int32)
    t = [x.cpu().numpy() for x in gd.fill_layer(cfg, 3, slot_expert)]
    hw = gi.HostWeights(cfg, 3)
    for s, e in enumerate(slot_expert):
        for m in (sm.MATRIX_GATE, sm.MATRIX_UP, sm.MATRIX_DOWN):
            codes, scales = hw.matrix(int(e), m)
            np.testing.assert_array_equal(t[2 * m][s], codes)
            np.testing.assert_array_equal(t[2 * m + 1][s], scales)
