"""The five synthetic workloads: shapes, dtypes, distributions and seeds.

Each workload stands in for a scale or accuracy setting the RACE Attention
pages describe without giving a shape (abstract on the fugumt page of
arXiv 2510.04008; the Italian gist.science page, "Sommario tecnico" section 3).
Seeds are 20251005 + workload index.  Temperature (beta) is 1.0 for all.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    P: int
    L: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    chunk: int
    backward: bool
    qk_dist: str        # "normal" or "mixture"
    beta: float = 1.0
    index: int = 0

    @property
    def seed(self) -> int:
        return 20251005 + self.index

    @property
    def R(self) -> int:
        return 1 << self.P

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.N

    def as_dict(self):
        d = asdict(self)
        d["seed"] = self.seed
        return d


WORKLOADS = [
    Workload("noncausal_fwd_n512_fp32", 1, 1, 512, 64, 2, 8, "f32", False, 512, False, "normal", index=0),
    # non-causal: the chunk only tiles the work (the configuration leaves it
    # free); 1024 measured fastest of 256 / 512 / 1024 (2.90 / 2.45 / 2.23 ms)
    Workload("noncausal_encoder_n4096", 32, 12, 4096, 64, 4, 32, "bf16", False, 1024, True, "normal", index=1),
    Workload("causal_lm_n32768_mixture", 8, 12, 32768, 64, 4, 32, "bf16", True, 256, True, "mixture", index=2),
    Workload("causal_long_n12M", 1, 4, 12_000_000, 64, 4, 16, "bf16", True, 1024, True, "normal", index=3),
    Workload("causal_extreme_n75M", 1, 1, 75_000_000, 64, 4, 8, "bf16", True, 2048, True, "normal", index=4),
]

BY_NAME = {w.name: w for w in WORKLOADS}
