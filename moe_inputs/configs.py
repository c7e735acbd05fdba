"""The five MoE-layer workloads this library is tested and measured on.

Each is one mixture-of-experts layer forward:  T tokens of width d, E routed
experts split into G equal groups (the "nodes" of node-limited routing), k
experts per token drawn from at most M groups, SwiGLU experts of width d_ff and
one shared expert of the same shape.

Shapes come from the pages:
  * DeepSeek-V3 uses node-limited routing with at most M=4 nodes over 256 routed
    experts (zenaique "MoE node-limited routing", "Real products"; deepnotes
    "DeepSeek-V3 671B: the real parallelism mesh", "The real cluster").
  * 8 routed + 1 shared expert per token at hidden width 7168 (zenaique, "Why
    all to all dominates MoE step time").
  * local batch 4 x sequence 4096 gives T = 16384 (deepnotes, "The artifact you
    actually inherit", the training block of the listed config).
  * 256 experts over 64 expert-parallel ranks = 4 experts per GPU, 32 per
    8-GPU node (deepnotes, "The real cluster").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int              # tokens
    d: int              # model width
    E: int              # routed experts
    G: int              # expert groups ("nodes")
    k: int              # routed experts per token
    M: int              # max groups per token
    d_ff: int           # expert hidden width
    dtype: str          # "f32" | "bf16" | "fp8": storage type of x, weights and the FFN
    n_shared: int = 1
    skew: bool = False                         # add a Zipf-ranked logit offset per expert
    local: Optional[Tuple[int, int]] = None    # [e_begin, e_end): this GPU's experts only
    seed: int = 0
    description: str = ""

    @property
    def gk(self) -> int:
        """Affinities summed per group score: ceil(k/M) (k/M when it divides)."""
        return -(-self.k // self.M)

    @property
    def group_size(self) -> int:
        return self.E // self.G

    @property
    def pairs(self) -> int:
        return self.T * self.k

    @property
    def e_begin(self) -> int:
        return 0 if self.local is None else self.local[0]

    @property
    def e_end(self) -> int:
        return self.E if self.local is None else self.local[1]

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    def validate(self) -> None:
        assert self.T >= 0 and self.d > 0 and self.E > 0 and self.G > 0
        assert self.E % self.G == 0, "groups must split the experts evenly"
        assert 1 <= self.M <= self.G
        assert 1 <= self.gk <= self.group_size
        assert 1 <= self.k <= self.M * self.group_size
        assert 0 <= self.e_begin <= self.e_end <= self.E


TINY = MoEConfig(
    name="tiny", T=256, d=64, E=16, G=4, k=4, M=2, d_ff=32, dtype="f32",
    description="fp32 correctness case, small enough for brute force")

FLASH = MoEConfig(
    name="flash", T=4096, d=2048, E=64, G=8, k=6, M=4, d_ff=2048, dtype="bf16",
    description="Flash-like layer, near-uniform load")

V3 = MoEConfig(
    name="v3", T=16384, d=7168, E=256, G=8, k=8, M=4, d_ff=2048, dtype="bf16",
    description="DeepSeek-V3-shaped layer, all 256 experts resident on one GPU")

V3_SKEW_EP0 = MoEConfig(
    name="v3_skew_ep0", T=16384, d=7168, E=256, G=8, k=8, M=4, d_ff=2048, dtype="bf16",
    skew=True, local=(0, 4),
    description="one expert-parallel rank's 4 experts under Zipf(1.2) routing skew, fp32 scatter-add output")

V3_SKEW_EP63 = MoEConfig(
    name="v3_skew_ep63", T=16384, d=7168, E=256, G=8, k=8, M=4, d_ff=2048, dtype="bf16",
    skew=True, local=(252, 256),
    description="the coldest expert-parallel rank's 4 experts (252-255) under the same Zipf(1.2) skew")

V3_FP8 = MoEConfig(
    name="v3_fp8", T=16384, d=7168, E=256, G=8, k=8, M=4, d_ff=2048, dtype="fp8",
    description="V3 shapes with e4m3 activations (1x128 fp32 scales) and weights (128x128 fp32 scales)")

CONFIGS = {c.name: c for c in (TINY, FLASH, V3, V3_SKEW_EP0, V3_SKEW_EP63, V3_FP8)}


def get(name: str) -> MoEConfig:
    return CONFIGS[name]


def flops_per_pair(cfg: MoEConfig) -> int:
    """Three d x d_ff matrices per SwiGLU expert, 2 flops per multiply-add."""
    return 6 * cfg.d * cfg.d_ff


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def log2_int(x: int) -> int:
    return int(math.log2(x))
