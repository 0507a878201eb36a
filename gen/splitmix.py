"""SplitMix64 counter generator (host side, numpy).

SplitMix64 is the generator of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators" (OOPSLA 2014), in the form later published
as the seeding generator of the xoshiro family: the state advances by the
odd constant GAMMA and every output is the state passed through the 64-bit
finaliser ``mix64``. Because the n-th output depends only on the seed and n,
any element of a stream can be produced independently; the device filler in
``gen/fill.hip`` implements the same definition and must produce the same
bytes.

Streams used for the synthetic expert weights
---------------------------------------------
Each (seed, layer, expert, matrix, kind) tuple owns one stream:

    stream_id = seed << 32 | layer << 24 | expert << 8 | matrix << 4 | kind
    s0        = mix64(stream_id)
    out(n)    = mix64(s0 + (n + 1) * GAMMA)            (mod 2**64)

matrix: 0 gate, 1 up, 2 down.  kind: 0 e2m1 code bytes, 1 UE8M0 scale bytes.

* Code byte i of a matrix (row-major, K contiguous) is byte (i mod 8),
  little-endian, of out(i div 8).  Both nibbles are therefore uniform on
  0..15.
* Scale byte i is 127 + emin + ((out(i) >> 32) * nrange >> 32) with
  nrange = 1 - emin, i.e. the exponent is uniform on [emin, 0] (Lemire's
  multiply-shift range reduction on the high 32 bits).

This module is input generation only; it holds none of the MoE arithmetic.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

MATRIX_GATE, MATRIX_UP, MATRIX_DOWN = 0, 1, 2
KIND_CODES, KIND_SCALES = 0, 1


def mix64_int(z: int) -> int:
    """The SplitMix64 finaliser on one Python int (reference form)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """Vectorised finaliser; uint64 arithmetic wraps mod 2**64 in numpy."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_id(seed: int, layer: int, expert: int, matrix: int, kind: int) -> int:
    assert 0 <= seed < 2**32 and 0 <= layer < 256 and 0 <= expert < 65536
    assert 0 <= matrix < 16 and 0 <= kind < 16
    return (seed << 32) | (layer << 24) | (expert << 8) | (matrix << 4) | kind


def stream_seed(seed: int, layer: int, expert: int, matrix: int, kind: int) -> int:
    return mix64_int(stream_id(seed, layer, expert, matrix, kind))


def outputs(s0: int, start: int, count: int) -> np.ndarray:
    """out(n) for n in [start, start+count) as uint64."""
    n = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(s0) + n * GAMMA
    return mix64(state)


def code_bytes(seed: int, layer: int, expert: int, matrix: int, nbytes: int) -> np.ndarray:
    """The first ``nbytes`` code bytes of one matrix (nbytes % 8 == 0)."""
    assert nbytes % 8 == 0
    s0 = stream_seed(seed, layer, expert, matrix, KIND_CODES)
    words = outputs(s0, 0, nbytes // 8)
    return words.astype("<u8", copy=False).view(np.uint8)


def scale_bytes(seed: int, layer: int, expert: int, matrix: int, count: int, emin: int) -> np.ndarray:
    """``count`` UE8M0 scale bytes with exponent uniform on [emin, 0]."""
    assert emin <= 0
    nrange = np.uint64(1 - emin)
    s0 = stream_seed(seed, layer, expert, matrix, KIND_SCALES)
    hi = outputs(s0, 0, count) >> np.uint64(32)
    with np.errstate(over="ignore"):
        r = (hi * nrange) >> np.uint64(32)
    return (np.int64(127 + emin) + r.astype(np.int64)).astype(np.uint8)
