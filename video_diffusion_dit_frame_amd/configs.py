"""Workloads: video-DiT attention layers (regions of cap = 64 tokens, the 8x8
cells when the sides divide, or 128).

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
    cap: int = 64

    @property
    def N(self) -> int:
        return self.F * self.Hv * self.Wv

    @property
    def R(self) -> int:
        """Regions: frames x ceil(Hv Wv / cap)."""
        return self.F * (-(-self.Hv * self.Wv // self.cap))

    @property
    def T(self) -> int:
        """Attention tiles of 64 slots: cap / 64 per region."""
        return self.R * self.cap // 64


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
    # the Wan-14B 720p layer at block capacity 128 (the capacity of the
    # paper's operator study): 30 regions of 128 tokens per frame
    "wan14b-720p-c128": Workload("wan14b-720p-c128", 1, 40, 128, 21, 48, 80, ((1000, 3000),), SEED0 + 2,
                                 cap=128),
    "sweep-wan14b-cfg": Workload("sweep-wan14b-cfg", 2, 40, 128, 21, 48, 80,
                                 ((500, 1500), (1000, 3000), (2000, 4000), (0, 6000), (10000, 0)),
                                 SEED0 + 4),
}
