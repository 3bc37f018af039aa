"""Workloads: video-DiT attention layers (8x8 spatial regions, 64 tokens).

Each entry: batch B, heads H, head_dim d, latent frames F x height Hv x width
Wv (tokens N = F*Hv*Wv in raster order), and budgets as (8-bit, MXFP4) shares
of the R^2 region pairs in basis points; the rest is skipped.
"""
from dataclasses import dataclass, field
from typing import List, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    F: int
    Hv: int
    Wv: int
    budgets: Tuple[Tuple[int, int], ...]
    seed: int
    outliers: bool = True
    lam: float = 0.2

    @property
    def N(self) -> int:
        return self.F * self.Hv * self.Wv

    @property
    def R(self) -> int:
        """Regions: frames x ceil(Hv Wv / 64)."""
        return self.F * (-(-self.Hv * self.Wv // 64))


SEED0 = 20260926

WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 4, 16, 16, ((2500, 2500),), SEED0 + 0, outliers=False),
    "wan1.3b": Workload("wan1.3b", 1, 12, 128, 21, 32, 48, ((1500, 3500),), SEED0 + 1),
    "wan14b-720p": Workload("wan14b-720p", 1, 40, 128, 21, 48, 80, ((1000, 3000),), SEED0 + 2),
    "hunyuan": Workload("hunyuan", 1, 24, 128, 33, 48, 80, ((1000, 3000),), SEED0 + 3),
    # latents whose sides are not multiples of 8 (ragged partitions): Wan2.1
    # at 832 x 480 and HunyuanVideo at 960 x 544 (spatial compression 16)
    "wan1.3b-480p": Workload("wan1.3b-480p", 1, 12, 128, 21, 30, 52, ((1500, 3500),), SEED0 + 5),
    "hunyuan-544p": Workload("hunyuan-544p", 1, 24, 128, 33, 34, 60, ((1000, 3000),), SEED0 + 6),
    "sweep-wan14b-cfg": Workload("sweep-wan14b-cfg", 2, 40, 128, 21, 48, 80,
                                 ((500, 1500), (1000, 3000), (2000, 4000), (0, 6000), (10000, 0)),
                                 SEED0 + 4),
}
