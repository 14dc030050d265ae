"""Seeded synthetic inputs for one rank's AllGather+GEMM, shared by the tests and the
benchmark.

This module holds the workload shapes and the random-number recipe only: no step of
the method is computed here. Both the fp64 oracle and the HIP path consume the
tensors it returns (the oracle after an exact upcast of the bf16 values to float64).

Recipe: torch.Generator('cpu').manual_seed(seed); draw the shards A [N, M_loc, K], then
the weight shard W [N_out, K], from randn in float32, in that order; round to bf16
(round to nearest even). The pages report AllGather+GEMM over gathered sizes M of
4K-32K rows (Figure 4) without K or N; these shapes take a hidden size of 8192 and a
4096-column weight shard per rank, and stand in for those problem sizes.
"""

from __future__ import annotations

from dataclasses import asdict, dataclass
from typing import Tuple

import torch


@dataclass(frozen=True)
class AgConfig:
    name: str
    n_ranks: int
    rank: int
    m_loc: int
    k: int
    n_out: int

    @property
    def m(self) -> int:
        return self.n_ranks * self.m_loc

    def as_dict(self):
        return asdict(self)


AG_CONFIGS = [
    AgConfig("ag_tiny_r1of4_M128x4_K256_N256", n_ranks=4, rank=1, m_loc=128, k=256, n_out=256),
    AgConfig("ag_r3of8_M2048x8_K8192_N4096", n_ranks=8, rank=3, m_loc=2048, k=8192, n_out=4096),
]
AG_CONFIG_BY_NAME = {c.name: c for c in AG_CONFIGS}
AG_TINY, AG_HEADLINE = AG_CONFIGS


def ag_sweep_config(m_total: int, n_ranks: int = 8, k: int = 8192, n_out: int = 4096) -> AgConfig:
    """The headline shape at another gathered size (the Figure 4 axis)."""
    return AgConfig(f"ag_r3of{n_ranks}_M{m_total // n_ranks}x{n_ranks}_K{k}_N{n_out}", n_ranks=n_ranks, rank=3,
                    m_loc=m_total // n_ranks, k=k, n_out=n_out)


def make_ag_inputs(cfg: AgConfig, seed: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """(a_shards [N, M_loc, K], w [N_out, K]) in bf16, drawn as the module recipe says."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    a = torch.randn((cfg.n_ranks, cfg.m_loc, cfg.k), generator=gen, dtype=torch.float32)
    w = torch.randn((cfg.n_out, cfg.k), generator=gen, dtype=torch.float32)
    return a.to(torch.bfloat16), w.to(torch.bfloat16)
