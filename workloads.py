"""Seeded synthetic inputs for the fused MoE dispatch + expert GEMM.

This module holds input generation only: shapes, distributions and seeds.  It
contains none of the routing, layout or GEMM arithmetic, and both the CPU
oracle and the HIP path consume what it returns.

The pages publish no workload ("mKernel UCCL fuses NVLink/RDMA/compute into
one persistent CUDA kernel", zubnet.ai, paragraph 4, notes that no
head-to-head numbers are given), so every input is synthetic:
  x      bf16, N(0, 1) rounded to nearest even
  Wr     fp32, N(0, 1/d)   (variance 1/d: logits of unit scale)
  W      bf16, N(0, 1/d)   [E_local, N, d], K contiguous (torch Linear layout)
  bias   only for the skewed workload: log2 of rank-Zipf(s=1.2) weights
  delays only for the wide-EP share: per-chunk arrival delay in microseconds,
         i.i.d. uniform integers in [0, 100]
Each tensor has its own torch CPU generator, seeded seed*1000 + tag
(x=1, Wr=2, W=3, delays=4), so draws do not depend on which other tensors are
generated.  Exact values depend on the torch version (recorded by the bench).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

TAG_X, TAG_WR, TAG_W, TAG_DELAY = 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (all sources together)
    d: int            # hidden size (GEMM K)
    E: int            # global experts the router scores
    k: int            # experts per token
    N: int            # expert output width (GEMM N)
    E_local: int      # experts held here: [e_begin, e_begin + E_local)
    e_begin: int = 0
    S: int = 1        # source shards (simulated peers); token t = s*rows_per_src + r
    chunk_rows: int = 0          # rows per arrival flag (0: no flags)
    zipf_bias: bool = False      # add log2 rank-Zipf(s=1.2) per-expert bias
    route_outside: bool = False  # routing done by the sources before payload arrival

    @property
    def rows_per_src(self) -> int:
        return self.T // self.S

    @property
    def r_cap(self) -> int:
        return self.T * min(self.k, self.E_local)


WORKLOADS = {
    # T=256, d=512, E=8, top-2, N=1024: the small case the oracle finishes in seconds.
    "tiny": Workload("tiny", T=256, d=512, E=8, k=2, N=1024, E_local=8),
    # Mixtral-shaped up-projection: T=4096, d=4096, E=8, top-2, N=14336, near-uniform load.
    "mixtral": Workload("mixtral", T=4096, d=4096, E=8, k=2, N=14336, E_local=8),
    # Fine-grained and skewed: T=8192, d=2048, E=64, top-6, N=1408, Zipf bias.
    "skewed": Workload("skewed", T=8192, d=2048, E=64, k=6, N=1408, E_local=64, zipf_bias=True),
    # One GPU's share of a wide expert-parallel layer: 8 sources x 2048 rows,
    # d=7168, 256 global experts, top-8, local experts 0..31, N=2048.
    "wide_ep": Workload("wide_ep", T=16384, d=7168, E=256, k=8, N=2048, E_local=32, S=8,
                        chunk_rows=128, route_outside=True),
    # Decode-shaped, weight-streaming bound: T=128, d=7168, 256 global experts,
    # top-8, local experts 0..31, N=2048.
    "decode": Workload("decode", T=128, d=7168, E=256, k=8, N=2048, E_local=32),
}


def _gen(seed: int, tag: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 1000 + tag)


def zipf_log2_bias(E: int, s: float = 1.2) -> np.ndarray:
    """fp32(log2(p_r)) with p_r = r^-s / sum_{q=1..E} q^-s, r = expert id + 1 (fp64 then rounded)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p = p / p.sum()
    return np.log2(p).astype(np.float32)


def make_x(wl: Workload, seed: int = 0) -> torch.Tensor:
    return torch.randn(wl.T, wl.d, generator=_gen(seed, TAG_X)).to(torch.bfloat16)


def make_w_router(wl: Workload, seed: int = 0) -> torch.Tensor:
    return torch.randn(wl.d, wl.E, generator=_gen(seed, TAG_WR)) / math.sqrt(wl.d)


def make_w_experts(wl: Workload, seed: int = 0) -> torch.Tensor:
    g = _gen(seed, TAG_W)
    out = torch.empty(wl.E_local, wl.N, wl.d, dtype=torch.bfloat16)
    scale = 1.0 / math.sqrt(wl.d)
    for e in range(wl.E_local):   # one expert at a time keeps the fp32 staging small
        out[e] = (torch.randn(wl.N, wl.d, generator=g) * scale).to(torch.bfloat16)
    return out


def make_bias(wl: Workload) -> Optional[torch.Tensor]:
    if not wl.zipf_bias:
        return None
    return torch.from_numpy(zipf_log2_bias(wl.E))


def make_delays_us(wl: Workload, seed: int = 0) -> Optional[torch.Tensor]:
    """Per-chunk arrival delays (uint32 microseconds), chunk c = s*chunks_per_src + j."""
    if wl.chunk_rows <= 0:
        return None
    n = wl.S * (-(-wl.rows_per_src // wl.chunk_rows))
    return torch.randint(0, 101, (n,), generator=_gen(seed, TAG_DELAY), dtype=torch.int64).to(torch.int32)


def make_inputs(wl: Workload, seed: int = 0, with_experts: bool = True) -> dict:
    """All inputs of one workload as CPU tensors."""
    out = dict(wl=wl, seed=seed, x=make_x(wl, seed), w_router=make_w_router(wl, seed),
               bias=make_bias(wl), delays_us=make_delays_us(wl, seed))
    if with_experts:
        out["w_experts"] = make_w_experts(wl, seed)
    return out


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of a workload with some sizes changed (parity cases at other sizes)."""
    return dataclasses.replace(wl, **changes)
