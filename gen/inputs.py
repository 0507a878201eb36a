"""Seeded synthetic inputs shaped like the pages' model.

The shapes come from the pages' description of the routed experts: 5120
hidden, expert width 2304, 384 routed experts per layer, 40 layers, every
expert stored as e2m1 codes with one UE8M0 scale per 32 weights (ds4-recipe /
GB10 spark README, "Why it is built this way").  Routing skew stands in for
the measured 40-layer routing trace that is not available: logits are
N(0,1) plus a per-expert Zipf(s) log-popularity bias.

Host draws (numpy PCG64 seeded with the config's seed), in this order:

1. if the config has a Zipf exponent s: ``perm = rng.permutation(E)``;
   expert e has rank perm[e] + 1 and bias ``-s * ln(rank)``;
2. for every layer, if only part of the experts is resident:
   ``sorted(rng.choice(E, n_resident, replace=False))`` -- slot j holds the
   j-th smallest resident expert id;
3. x: ``rng.standard_normal((T, H))`` rounded to float32, then to bf16 with
   round-to-nearest-even (stored as uint16 bit patterns);
4. for every layer: ``rng.standard_normal((T, E)) + bias`` rounded to float32.

Extra logit sets (used to rotate the experts a timing loop touches) come from
a second generator PCG64([seed, 1 + layer]) with the same bias.  The router
gate rows W_r (the projection upstream of the router) come from a third,
PCG64([seed, 1000 + layer]), see router_weights.

Weight bytes come from the SplitMix64 streams documented in gen/splitmix.py,
keyed by expert id (not slot), so an expert's bytes do not depend on which
slot it occupies.

No MoE arithmetic lives here.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import splitmix as sm


@dataclass(frozen=True)
class Config:
    name: str
    H: int          # hidden size
    I: int          # expert width
    E: int          # routed experts per layer
    k: int          # experts per token
    T: int          # tokens
    emin: int       # scale exponents uniform on [emin, 0]
    seed: int
    zipf: float | None = None
    layers: int = 1
    resident: int | None = None   # experts resident per layer (None: all)
    desc: str = field(default="", compare=False)

    @property
    def slots(self) -> int:
        return self.E if self.resident is None else self.resident

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert: three matrices of codes plus scales."""
        return 3 * self.H * self.I // 2 + 3 * self.H * self.I // 32


CONFIGS = {
    "tiny": Config("tiny", 256, 128, 8, 2, 4, -4, 1001,
                   desc="tiny layer: H=256 I=128 E=8 top-2 T=4"),
    "decode1": Config("decode1", 5120, 2304, 384, 8, 1, -6, 1002,
                      desc="single-layer decode, batch 1, 384 experts resident"),
    "verify16": Config("verify16", 5120, 2304, 384, 8, 16, -6, 1003, zipf=1.1,
                       desc="single-layer decode, 16 tokens, Zipf(1.1) routing bias"),
    "prefill4096": Config("prefill4096", 5120, 2304, 384, 8, 4096, -6, 1004, zipf=1.1,
                          desc="single-layer prefill chunk, 4096 tokens, Zipf(1.1)"),
    "chain40": Config("chain40", 5120, 2304, 384, 8, 1, -6, 1005, layers=40, resident=154,
                      desc="40-layer chained decode, 154 of 384 experts resident per layer"),
}


def custom(name: str, H: int, I: int, E: int, k: int, T: int, *, emin: int = -6,
           seed: int = 7, zipf: float | None = None, layers: int = 1,
           resident: int | None = None) -> Config:
    return Config(name, H, I, E, k, T, emin, seed, zipf, layers, resident)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + r) >> np.uint64(16)).astype(np.uint16)


@dataclass
class HostInputs:
    cfg: Config
    x_bf16: np.ndarray                 # uint16 [T][H]
    logits: list[np.ndarray]           # per layer float32 [T][E]
    resident: list[np.ndarray]         # per layer int64 [slots] expert ids, ascending
    expert_to_slot: list[np.ndarray]   # per layer int32 [E]; -1 = not resident
    bias: np.ndarray                   # float64 [E]


def host_inputs(cfg: Config) -> HostInputs:
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    bias = np.zeros(cfg.E)
    if cfg.zipf is not None:
        perm = rng.permutation(cfg.E)
        bias = -cfg.zipf * np.log(perm + 1.0)
    resident, e2s = [], []
    for _ in range(cfg.layers):
        if cfg.resident is None:
            res = np.arange(cfg.E, dtype=np.int64)
        else:
            res = np.sort(rng.choice(cfg.E, cfg.resident, replace=False)).astype(np.int64)
        table = np.full(cfg.E, -1, dtype=np.int32)
        table[res] = np.arange(len(res), dtype=np.int32)
        resident.append(res)
        e2s.append(table)
    x = f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
    logits = [(rng.standard_normal((cfg.T, cfg.E)) + bias).astype(np.float32)
              for _ in range(cfg.layers)]
    return HostInputs(cfg, x, logits, resident, e2s, bias)


def logit_sets(cfg: Config, bias: np.ndarray, n: int, layer: int = 0) -> np.ndarray:
    """``n`` further logit sets float32 [n][T][E] for rotating a timing loop."""
    rng = np.random.Generator(np.random.PCG64([cfg.seed, 1 + layer]))
    return (rng.standard_normal((n, cfg.T, cfg.E)) + bias).astype(np.float32)


def router_weights(cfg: Config, layer: int = 0) -> np.ndarray:
    """Router gate rows W_r as bf16 bit patterns [E][H].

    Draws ``rng.standard_normal((E, H)) / sqrt(H)`` from PCG64([seed, 1000 +
    layer]), rounded to float32 and then to bf16 (nearest even).  With x ~
    N(0,1) the projected logits have unit variance, like the configs' logits.
    """
    rng = np.random.Generator(np.random.PCG64([cfg.seed, 1000 + layer]))
    w = rng.standard_normal((cfg.E, cfg.H)) / np.sqrt(cfg.H)
    return f32_to_bf16_bits(w.astype(np.float32))


def router_bias(hi: "HostInputs") -> np.ndarray | None:
    """The config's per-expert popularity bias as float32 [E], or None without one."""
    return hi.bias.astype(np.float32) if hi.cfg.zipf is not None else None


# cb3 experts: index bytes from the SplitMix code streams of matrices 8 + m
# (gate 8, up 9, down 10), codebooks from PCG64([seed, 2000 + layer, expert, m]).
CB3_MATRIX_BASE = 8


def cb3_codebook(cfg: Config, layer: int, expert: int, matrix: int) -> np.ndarray:
    """One matrix's per-row codebooks as bf16 bits [rows][8]: N(0,1)/8 rounded
    to float32, then to bf16 (nearest even)."""
    rows = cfg.I if matrix in (sm.MATRIX_GATE, sm.MATRIX_UP) else cfg.H
    rng = np.random.Generator(np.random.PCG64([cfg.seed, 2000 + layer, expert, matrix]))
    return f32_to_bf16_bits((rng.standard_normal((rows, 8)) / 8).astype(np.float32))


class HostCb3Weights:
    """Host copy of one layer's synthetic cb3 experts, generated on demand.

    Layouts (row-major, K contiguous): index bytes gate/up [I][3H/8], down
    [H][3I/8]; codebooks gate/up [I][8], down [H][8] bf16 bits.
    """

    def __init__(self, cfg: Config, layer: int = 0):
        self.cfg, self.layer = cfg, layer
        self._cache: dict[tuple[int, int], tuple[np.ndarray, np.ndarray]] = {}

    def matrix(self, expert: int, matrix: int) -> tuple[np.ndarray, np.ndarray]:
        key = (expert, matrix)
        if key not in self._cache:
            c = self.cfg
            rows, K = (c.I, c.H) if matrix in (sm.MATRIX_GATE, sm.MATRIX_UP) else (c.H, c.I)
            q = sm.code_bytes(c.seed, self.layer, expert, CB3_MATRIX_BASE + matrix, rows * K * 3 // 8)
            self._cache[key] = (q.reshape(rows, K * 3 // 8), cb3_codebook(c, self.layer, expert, matrix))
        return self._cache[key]


class HostWeights:
    """Host copy of one layer's synthetic expert bytes, generated on demand.

    Layouts (row-major, K contiguous; element 2c of a row in the low nibble
    of byte c):
      gate, up : codes [I][H/2], scales [I][H/32]
      down     : codes [H][I/2], scales [H][I/32]
    """

    def __init__(self, cfg: Config, layer: int = 0):
        self.cfg, self.layer = cfg, layer
        self._cache: dict[tuple[int, int], tuple[np.ndarray, np.ndarray]] = {}

    def shape(self, matrix: int) -> tuple[int, int]:
        c = self.cfg
        return (c.I, c.H) if matrix in (sm.MATRIX_GATE, sm.MATRIX_UP) else (c.H, c.I)

    def matrix(self, expert: int, matrix: int) -> tuple[np.ndarray, np.ndarray]:
        key = (expert, matrix)
        if key not in self._cache:
            rows, K = self.shape(matrix)
            c = self.cfg
            codes = sm.code_bytes(c.seed, self.layer, expert, matrix, rows * K // 2)
            scales = sm.scale_bytes(c.seed, self.layer, expert, matrix, rows * K // 32, c.emin)
            self._cache[key] = (codes.reshape(rows, K // 2), scales.reshape(rows, K // 32))
        return self._cache[key]

    def drop(self) -> None:
        self._cache.clear()
