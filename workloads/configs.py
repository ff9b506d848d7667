"""The five synthetic workloads and their integer structure.

Shapes and distributions follow the workload list this library is measured on
(the PLoRA page's setting: many LoRA jobs of different ranks and token counts
over one frozen base, PLoRA: Efficient Concurrent LoRA Training for Large
Language Models, §2.4 and §11.2.1).  Where the description leaves a choice
open the reading taken is written next to the draw.

Token counts and ranks are drawn once with ``numpy.random.default_rng(seed)``
and frozen into ``workloads/frozen/<name>_s<seed>.json`` by ``freeze.py`` so
results never depend on numpy's sampler version.  ``load_workload`` reads the
frozen file when it exists and draws otherwise.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field, asdict
from typing import List

import numpy as np

FROZEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "frozen")

WORKLOAD_NAMES = ("tiny_fp32", "llama7b_proj", "llama3_8b_layer", "nano_stress", "mlp70b_pair")

# Value distributions (standard deviations).  X and dY ~ N(0, 1); W0 ~ N(0, 0.02);
# B_i ~ N(0, 0.01); A_i ~ N(0, 1/d_in) read as a fan-in variance, std = d_in**-0.5.
STD_X = 1.0
STD_DY = 1.0
STD_W0 = 0.02
STD_B = 0.01


def std_a(d_in: int) -> float:
    return float(d_in) ** -0.5


@dataclass
class Projection:
    name: str
    d_in: int
    d_out: int


@dataclass
class Workload:
    name: str
    dtype: str                      # "fp32" or "bf16"
    projections: List[Projection]
    ranks: List[int]
    tokens: List[int]
    n_streams: int = 1
    seed: int = 0
    note: str = ""
    scales: List[float] = field(default_factory=list)

    def __post_init__(self):
        if not self.scales:
            # s_i = 16 / r_i, exact in fp32 for power-of-two ranks.
            self.scales = [16.0 / r for r in self.ranks]

    @property
    def n(self) -> int:
        return len(self.ranks)

    @property
    def T(self) -> int:
        return int(sum(self.tokens))

    def seg_offsets(self) -> np.ndarray:
        o = np.zeros(self.n + 1, dtype=np.int64)
        o[1:] = np.cumsum(np.asarray(self.tokens, dtype=np.int64))
        return o

    def to_json(self) -> str:
        d = asdict(self)
        return json.dumps(d, indent=1)

    @staticmethod
    def from_json(s: str) -> "Workload":
        d = json.loads(s)
        d["projections"] = [Projection(**p) for p in d["projections"]]
        return Workload(**d)

    def scaled_down(self, max_tokens: int, max_dim: int = 0) -> "Workload":
        """Same adapter/rank structure with token counts shrunk proportionally
        (every adapter keeps at least one token unless it had none) and, if
        ``max_dim`` is set, each projection dimension capped at ``max_dim``."""
        T = self.T
        if T > max_tokens:
            toks = [max(1 if t > 0 else 0, (t * max_tokens) // T) for t in self.tokens]
        else:
            toks = list(self.tokens)
        projs = self.projections
        if max_dim:
            projs = [Projection(p.name, min(p.d_in, max_dim), min(p.d_out, max_dim)) for p in projs]
        return Workload(self.name + "_small", self.dtype, projs, list(self.ranks), toks,
                        self.n_streams, self.seed, self.note, list(self.scales))


def largest_remainder(weights: np.ndarray, total: int) -> List[int]:
    """Integer counts proportional to ``weights`` summing to ``total``, at
    least 1 each.  Floors first; the shortfall goes one unit at a time to the
    largest fractional parts (ties to the lower index); any zero count is then
    raised to 1 by taking one unit from the currently largest count (ties to
    the lower index)."""
    w = np.asarray(weights, dtype=np.float64)
    q = w / w.sum() * total
    base = np.floor(q).astype(np.int64)
    frac = q - base
    short = int(total - base.sum())
    order = sorted(range(len(w)), key=lambda i: (-frac[i], i))
    for i in order[:short]:
        base[i] += 1
    for i in range(len(w)):
        if base[i] == 0:
            j = max(range(len(w)), key=lambda k: (base[k], -k))
            base[j] -= 1
            base[i] = 1
    assert int(base.sum()) == total
    return [int(x) for x in base]


def draw_workload(name: str, seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    if name == "tiny_fp32":
        # d_in = d_out = 256, two adapters of ranks 4 and 8, 64 tokens each, fp32.
        return Workload(name, "fp32", [Projection("proj", 256, 256)], [4, 8], [64, 64],
                        seed=seed, note="tiny fp32 parity workload")
    if name == "llama7b_proj":
        # One 4096x4096 projection, four adapters; ranks and token counts paired
        # in the listed order.
        return Workload(name, "bf16", [Projection("proj", 4096, 4096)], [8, 16, 32, 64],
                        [512, 1024, 2048, 4096], seed=seed,
                        note="Llama-7B-shaped projection, 4 adapters")
    if name == "llama3_8b_layer":
        # Seven projections of one Llama-3-8B-shaped decoder layer; the same 16
        # adapters (ranks, token counts) on every projection.  Ranks i.i.d.
        # uniform over {8,16,32,64,128}; token counts i.i.d. uniform in
        # [256, 4096] inclusive.
        ranks = [int(x) for x in rng.choice([8, 16, 32, 64, 128], size=16)]
        toks = [int(x) for x in rng.integers(256, 4096, size=16, endpoint=True)]
        projs = [Projection("q", 4096, 4096), Projection("k", 4096, 1024),
                 Projection("v", 4096, 1024), Projection("o", 4096, 4096),
                 Projection("gate", 4096, 14336), Projection("up", 4096, 14336),
                 Projection("down", 14336, 4096)]
        return Workload(name, "bf16", projs, ranks, toks, seed=seed,
                        note="Llama-3-8B decoder layer, 7 projections, 16 adapters")
    if name == "nano_stress":
        # 64 adapters on a 4096x14336 up-projection; ranks i.i.d. uniform over
        # {4,...,256}; token counts from i.i.d. Zipf(1.1) draws truncated to
        # [1, 32768] by rejection, then scaled to total 32768 by largest
        # remainder with at least one token each.
        ranks = [int(x) for x in rng.choice([4, 8, 16, 32, 64, 128, 256], size=64)]
        draws = []
        while len(draws) < 64:
            z = int(rng.zipf(1.1))
            if z <= 32768:
                draws.append(z)
        toks = largest_remainder(np.asarray(draws, dtype=np.float64), 32768)
        return Workload(name, "bf16", [Projection("up", 4096, 14336)], ranks, toks, seed=seed,
                        note="rank-aware nano-batch stress, Zipf(1.1) token counts")
    if name == "mlp70b_pair":
        # Two 70B-shaped MLP projections; 32 adapters with ranks i.i.d. uniform
        # over {16,32,64,128,256}; 65536 tokens split by log-normal(0, 1)
        # weights with largest-remainder rounding; four HIP streams.
        ranks = [int(x) for x in rng.choice([16, 32, 64, 128, 256], size=32)]
        w = rng.lognormal(0.0, 1.0, size=32)
        toks = largest_remainder(w, 65536)
        return Workload(name, "bf16", [Projection("up", 8192, 28672), Projection("down", 28672, 8192)],
                        ranks, toks, n_streams=4, seed=seed,
                        note="70B-shaped MLP pair, log-normal token split, 4 streams")
    raise KeyError(name)


def frozen_path(name: str, seed: int) -> str:
    return os.path.join(FROZEN_DIR, f"{name}_s{seed}.json")


def load_workload(name: str, seed: int = 0) -> Workload:
    p = frozen_path(name, seed)
    if os.path.exists(p):
        with open(p) as f:
            return Workload.from_json(f.read())
    return draw_workload(name, seed)
