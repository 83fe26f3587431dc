"""Workload definitions (sizes and distributions only).

C1  single expert linear, no routing: X 16x512 ~N(0,1), W 1024x512 ~N(0,0.02),
    int3 group 64 along K, compensator A 512x16, B 16x1024 ~N(0,0.01).
C2  Mixtral-8x7B-shaped MoE FFN at decode: 16 tokens, hidden 4096, ffn 14336,
    8 experts, top-2 with renormalised softmax, ranks drawn from {16,32,64}.
C3  the same layer at prefill: 4096 tokens.
C4  DeepSeekMoE-16B-shaped layer: hidden 2048, 64 routed experts of ffn 1408,
    top-6 (plain softmax probabilities), 2 always-on shared experts (rank 32),
    256 tokens, Zipf(1.2)-skewed router logits, ranks from {8,16,32}.
C5  32 Mixtral-shaped blocks, decode batch sweep 1/8/32/64.

sigma values are standard deviations.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class LinearConfig:
    name: str
    cfg_id: int
    M: int
    N: int
    K: int
    rank: int
    group: int = 64
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    lr_sigma: float = 0.01


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    T: int                 # tokens
    H: int                 # hidden
    F: int                 # expert ffn width
    E: int                 # routed experts
    k: int                 # top-k
    S: int = 0             # shared (always-on) experts
    ranks: Tuple[int, ...] = (16, 32, 64)
    shared_rank: int = 32
    renormalize: bool = True
    zipf_alpha: float = 0.0   # 0 -> plain N(0,1) logits
    layers: int = 1
    group: int = 64
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    lr_sigma: float = 0.01
    logit_sigma: float = 1.0

    @property
    def slots(self) -> int:
        return self.k + self.S

    @property
    def P(self) -> int:
        return self.T * self.slots

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


C1 = LinearConfig("C1_single_linear", 1, M=16, N=1024, K=512, rank=16)
C2 = MoEConfig("C2_mixtral_decode", 2, T=16, H=4096, F=14336, E=8, k=2)
C3 = MoEConfig("C3_mixtral_prefill", 3, T=4096, H=4096, F=14336, E=8, k=2)
C4 = MoEConfig("C4_deepseekmoe16b", 4, T=256, H=2048, F=1408, E=64, k=6, S=2,
               ranks=(8, 16, 32), shared_rank=32, renormalize=False,
               zipf_alpha=1.2)
C5 = MoEConfig("C5_mixtral_stack32", 5, T=64, H=4096, F=14336, E=8, k=2,
               layers=32)
C5_BATCHES = (1, 8, 32, 64)

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}


def get_config(name: str):
    return CONFIGS[name]
