"""The five synthetic MoE-layer workloads (shapes, distributions, seeds).

Shapes follow the K-EXAONE layer: hidden 6144, expert intermediate 2048,
top-8 routing over 80 (REAP-pruned) or 128 (unpruned) routed experts.  The
token counts stand in for the workloads the pages describe: 16 tokens is a
decode batch of a few streams with their speculative rows, 8192 tokens is the
calibration maximum sequence length, 32768 tokens is the 32K context point.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class WeightSet:
    """One set of expert + router weights shared by the workloads that name it."""

    name: str
    seed_key: int
    E: int
    H: int
    I: int
    outliers: bool = False  # 0.5% of entries replaced by Laplace(0, 0.15) draws
    n_cal: int = 512  # calibration tokens for the static activation global scales


@dataclass(frozen=True)
class LayerConfig:
    index: int
    name: str
    weights: WeightSet
    k: int
    T: int
    bias: str  # "uniform": U(-0.1, 0.1); "zipf": fitted so expert counts follow Zipf(1.1)
    reap: bool
    bound: str  # which roofline bounds the layer at this shape: "latency", "hbm", "mfma"
    rsf: float = 2.5

    @property
    def E(self) -> int:
        return self.weights.E

    @property
    def H(self) -> int:
        return self.weights.H

    @property
    def I(self) -> int:
        return self.weights.I

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def describe(self) -> str:
        return (f"E{self.E} top-{self.k} H{self.H} I{self.I} T{self.T}"
                + (" zipf-skewed" if self.bias == "zipf" else "")
                + (" outliers" if self.weights.outliers else "")
                + (" +REAP" if self.reap else ""))


TINY8 = WeightSet("tiny8", 0x10, E=8, H=256, I=128)
E80 = WeightSet("e80", 0x50, E=80, H=6144, I=2048)
E128_OUTLIER = WeightSet("e128_outlier", 0x80, E=128, H=6144, I=2048, outliers=True)

CONFIGS = (
    LayerConfig(0, "tiny", TINY8, k=2, T=64, bias="uniform", reap=True, bound="latency"),
    LayerConfig(1, "decode", E80, k=8, T=16, bias="uniform", reap=False, bound="hbm"),
    LayerConfig(2, "prefill_zipf", E80, k=8, T=8192, bias="zipf", reap=False, bound="mfma"),
    LayerConfig(3, "outlier_128e", E128_OUTLIER, k=8, T=8192, bias="uniform", reap=False, bound="mfma"),
    LayerConfig(4, "long_reap", E80, k=8, T=32768, bias="uniform", reap=True, bound="mfma"),
)

WEIGHT_SETS = {w.name: w for w in (TINY8, E80, E128_OUTLIER)}


def config(i: int) -> LayerConfig:
    return CONFIGS[i]


def by_name(name: str) -> LayerConfig:
    """The workload with this name (tiny, decode, prefill_zipf, outlier_128e, long_reap)."""
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
