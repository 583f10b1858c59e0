"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module draws random numbers and picks sample rows; it holds none of the
attention arithmetic.  Everything is generated on the CPU with a
torch.Generator so the same seed gives the same bytes on every machine.

Draw order for a workload (seed = workload.seed): Q, then K, then V, all fp32;
then, for the "stress" distribution only, the set of key token rows that are
scaled by 8.  bf16 workloads round the fp32 draws to bfloat16 (round to nearest
even, torch's cast).  Scaling by 8 is a power of two, so it is exact before the
cast.

Distributions:
  normal : Q, K, V ~ N(0, 1)
  stress : Q ~ N(0, 1); K ~ N(0, 1) with round(0.01 * N) token rows (shared by
           every kv head and every channel) multiplied by 8; V ~ U(-1, 1) drawn
           as 2 * rand - 1.
"""
from __future__ import annotations

import hashlib
from typing import Dict, Optional

import torch

from .workloads import Workload

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def draw_qkv(B: int, nq: int, nkv: int, Hq: int, Hkv: int, d: int, seed: int,
             dtype: str = "bf16", dist: str = "normal") -> Dict[str, torch.Tensor]:
    """Q [B, nq, Hq, d], K and V [B, nkv, Hkv, d] on the CPU, in `dtype`."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, nq, Hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, nkv, Hkv, d), generator=g, dtype=torch.float32)
    if dist == "normal":
        v = torch.randn((B, nkv, Hkv, d), generator=g, dtype=torch.float32)
    elif dist == "stress":
        v = 2.0 * torch.rand((B, nkv, Hkv, d), generator=g, dtype=torch.float32) - 1.0
        nrows = int(round(0.01 * nkv))
        rows = torch.randperm(nkv, generator=g)[:nrows]
        k[:, rows] *= 8.0
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    t = _DT[dtype]
    return {"q": q.to(t).contiguous(), "k": k.to(t).contiguous(), "v": v.to(t).contiguous()}


def stress_rows(nkv: int, seed: int, B: int, nq: int, Hq: int, Hkv: int, d: int) -> torch.Tensor:
    """The token rows draw_qkv(..., dist="stress") scaled by 8 (replays the draw order)."""
    g = torch.Generator("cpu").manual_seed(seed)
    torch.randn((B, nq, Hq, d), generator=g)
    torch.randn((B, nkv, Hkv, d), generator=g)
    torch.rand((B, nkv, Hkv, d), generator=g)
    return torch.randperm(nkv, generator=g)[: int(round(0.01 * nkv))]


def workload_inputs(w: Workload) -> Dict[str, torch.Tensor]:
    """Inputs of a workload.

    When every rank of the ring is computed (the tiny workload) Q covers the
    whole sequence [B, N, Hq, d] and each rank takes its slice with local_q().
    Otherwise Q is drawn as the single computed rank's local block
    [B, N/P, Hq, d] (for P = 1 that is the whole sequence).
    """
    nq = w.N if len(w.ranks) == w.P else w.nq
    return draw_qkv(w.B, nq, w.N, w.Hq, w.Hkv, w.d, w.seed, w.dtype, w.dist)


def local_q(w: Workload, q: torch.Tensor, rank: int) -> torch.Tensor:
    if q.shape[1] == w.nq:
        return q
    return q[:, rank * w.nq:(rank + 1) * w.nq]


def sha256(t: torch.Tensor) -> str:
    x = t.contiguous()
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    return hashlib.sha256(x.numpy().tobytes()).hexdigest()


def sample_rows(B: int, Hq: int, nq: int, seed: int, tile: int = 128,
                extra_tiles: Optional[list] = None) -> torch.Tensor:
    """Rows (b, h, i) checked at full size.

    Every row of the first and last q-tiles of heads 0 and Hq-1 (plus any
    `extra_tiles`), and one seeded-random row per (q-tile, head, batch).
    Returns an int64 tensor [n, 3], sorted and unique.
    """
    g = torch.Generator("cpu").manual_seed(seed + 1000)
    ntile = (nq + tile - 1) // tile
    tiles = {0, ntile - 1}
    if extra_tiles:
        tiles.update(t for t in extra_tiles if 0 <= t < ntile)
    out = []
    for b in range(B):
        for h in sorted({0, Hq - 1}):
            for t in sorted(tiles):
                for i in range(t * tile, min(nq, (t + 1) * tile)):
                    out.append((b, h, i))
        for h in range(Hq):
            for t in range(ntile):
                lo, hi = t * tile, min(nq, (t + 1) * tile)
                i = lo + int(torch.randint(hi - lo, (1,), generator=g))
                out.append((b, h, i))
    rows = torch.tensor(sorted(set(out)), dtype=torch.int64)
    return rows
