"""The five synthetic workloads of the rank-share ring-attention path.

Each workload is one rank's share of ring (blockwise) attention as described on
the glossary page "sequence parallelism transformers", section "Ring Attention"
(items "Block-Wise Attention" and "Computation"): a local query block of
N/P tokens attends to the P key/value blocks of the sequence.  The Ulysses
workload is the "Ulysses Sequence Parallelism" section's head-parallel layout
(item "Attention Computation"): all N tokens for a subset of heads, i.e. the same
computation with P = 1.

Shapes use the [batch, seq, heads, head_dim] layout, sequence on dim 1, as the
mvp-engine sequence-parallel skill page fixes for [batch, seq, hidden]
activations (section "Bind on the same top-level model class").

This module holds sizes only; no arithmetic of the method.
"""
from __future__ import annotations

import dataclasses
from typing import Tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": element type of q, k, v
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int                # total sequence length (all P blocks)
    P: int                # ring size
    ranks: Tuple[int, ...]  # ranks whose share is computed
    causal: bool
    dist: str             # "normal" (Q,K,V ~ N(0,1)) or "stress" (see inputs.py)
    seed: int

    @property
    def nq(self) -> int:
        return self.N // self.P

    @property
    def nkv(self) -> int:
        return self.N // self.P

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    def shrunk(self, factor: int = 16) -> "Workload":
        """Same heads, head_dim, ring size, rank and distribution; N divided by factor."""
        assert self.N % (factor * self.P) == 0
        return dataclasses.replace(self, name=self.name + f"_div{factor}", N=self.N // factor)


TINY_F32 = Workload("tiny_f32_noncausal", "f32", 1, 2, 2, 64, 512, 4, (0, 1, 2, 3), False, "normal", 1)
RANK7_BF16 = Workload("rank7_of_8_bf16_causal", "bf16", 1, 32, 32, 128, 32768, 8, (7,), True, "normal", 2)
GQA_BF16 = Workload("gqa_rank15_of_16_bf16_causal", "bf16", 1, 32, 8, 128, 131072, 16, (15,), True, "normal", 3)
ULYSSES_BF16 = Workload("ulysses_4heads_bf16_causal", "bf16", 1, 4, 4, 128, 65536, 1, (0,), True, "normal", 4)
STRESS_BF16 = Workload("stress_rank31_of_32_bf16_causal", "bf16", 1, 8, 8, 128, 262144, 32, (31,), True, "stress", 5)

ALL = (TINY_F32, RANK7_BF16, GQA_BF16, ULYSSES_BF16, STRESS_BF16)
BY_NAME = {w.name: w for w in ALL}
