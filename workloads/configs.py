"""The named workloads: shapes, precision, block size, top-p and the input recipe.

The five named workloads are the shapes the FVAttn review (video DiT attention
with top-p routing) and the FlashAttention review motivate: a tiny fp32 case,
a dense bf16 case, two video-DiT-shaped sparse cases at 21x30x52 latent
patches and one long-video case at 33x45x80 latent patches.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # integer id mixed into every seed
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    block: int
    dtype: str               # "bf16" or "f32"
    top_p: float
    structured: bool         # Q/K = N(0,1) + a_h * E  (else iid N(0,1))
    grid: Optional[Tuple[int, int, int]] = None   # (T, Y, X) token grid
    gain: str = "uniform"    # a_h law: "uniform" U[lo,hi] or "loguniform"
    gain_range: Tuple[float, float] = (0.5, 4.0)
    embed_rms: float = 0.5   # RMS of each row of E

    @property
    def num_blocks(self) -> int:
        return math.ceil(self.seq_len / self.block)

    @property
    def units(self) -> int:
        return self.batch * self.heads * self.num_blocks

    def shape(self):
        return (self.batch, self.heads, self.seq_len, self.head_dim)

    def describe(self) -> str:
        return (f"{self.name}: B={self.batch} H={self.heads} N={self.seq_len} "
                f"d={self.head_dim} {self.dtype} block={self.block} p={self.top_p}")


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", 1, 1, 2, 256, 64, 64, "f32", 0.9, False),
    "dense-4k": Workload("dense-4k", 2, 1, 16, 4096, 128, 64, "bf16", 1.0, False),
    "video-32k": Workload("video-32k", 3, 1, 40, 32760, 128, 64, "bf16", 0.9, True,
                          grid=(21, 30, 52), gain="uniform", gain_range=(0.5, 4.0)),
    "skewed-32k": Workload("skewed-32k", 4, 1, 40, 32760, 128, 64, "bf16", 0.95, True,
                           grid=(21, 30, 52), gain="loguniform", gain_range=(0.25, 8.0)),
    "video-119k": Workload("video-119k", 5, 1, 24, 118800, 128, 128, "bf16", 0.9, True,
                           grid=(33, 45, 80), gain="uniform", gain_range=(0.5, 4.0)),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def custom_workload(batch, heads, seq_len, head_dim, block, dtype="bf16", top_p=0.9,
                    structured=True, grid=None, gain="uniform", gain_range=(0.5, 4.0),
                    wid=100, name=None) -> Workload:
    """A workload of any shape with the same recipe (used for small parity cases)."""
    if structured and grid is None:
        x = 13
        y = 7
        t = math.ceil(seq_len / (x * y))
        grid = (t, y, x)
    return Workload(name or f"custom-{batch}x{heads}x{seq_len}x{head_dim}-b{block}-{dtype}",
                    wid, batch, heads, seq_len, head_dim, block, dtype, top_p, structured,
                    grid=grid, gain=gain, gain_range=gain_range)
