"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds the workload shapes and the random-number recipe only: no step of the
attention method is computed here. Both the fp64 oracle and the HIP path consume the
tensors it returns (the oracle after an exact upcast of the bf16 values to float64).

Recipe (the pages publish no dataset for Ring Attention; these shapes stand in for their
workloads: 16 ranks, long sequences of the sizes swept in Fig. 3 of the mKernel paper):
  torch.Generator('cpu').manual_seed(seed); draw Q [Lq, Hq, D] then KV [N, 2, Lk, Hkv, D]
  from randn in float32, in that order; multiply Q and K by ``qk_mult`` (exact in bf16:
  2.0 for the peaky long-context workload, else 1.0); round to bf16 (round to nearest even).
"""

from __future__ import annotations

from dataclasses import dataclass, asdict
from typing import Tuple

import torch


@dataclass(frozen=True)
class RingConfig:
    name: str
    rank: int
    n_chunks: int
    lq: int
    lk: int
    hq: int
    hkv: int
    d: int
    causal: bool
    qk_mult: float = 1.0

    @property
    def gqa_ratio(self) -> int:
        return self.hq // self.hkv

    @property
    def n_steps(self) -> int:
        return self.rank + 1 if self.causal else self.n_chunks

    def as_dict(self):
        return asdict(self)


# The five workloads: a tiny D = 64 case, the small causal MHA case, the per-rank share
# of a 64K-token causal GQA sequence over 16 ranks (the headline shape), the same at 128K
# tokens with scores doubled, and a 32K-token MHA D = 64 ring.
CONFIGS = [
    RingConfig("tiny_r0of4_L128_h2_d64_nc", rank=0, n_chunks=4, lq=128, lk=128, hq=2, hkv=2, d=64, causal=False),
    RingConfig("small_r3of8_L1024_h16_d128_causal", rank=3, n_chunks=8, lq=1024, lk=1024, hq=16, hkv=16, d=128,
               causal=True),
    RingConfig("seq64k_r15of16_L4096_h32kv8_d128_causal", rank=15, n_chunks=16, lq=4096, lk=4096, hq=32, hkv=8,
               d=128, causal=True),
    RingConfig("seq128k_r15of16_L8192_h32kv8_d128_causal_qk2", rank=15, n_chunks=16, lq=8192, lk=8192, hq=32,
               hkv=8, d=128, causal=True, qk_mult=2.0),
    RingConfig("seq32k_r7of16_L2048_h64_d64_nc", rank=7, n_chunks=16, lq=2048, lk=2048, hq=64, hkv=64, d=64,
               causal=False),
]

CONFIG_BY_NAME = {c.name: c for c in CONFIGS}
TINY, SMALL, SEQ64K, SEQ128K, SEQ32K_D64 = CONFIGS


def make_inputs(cfg: RingConfig, seed: int, device: str = "cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """(q [Lq, Hq, D], kv_chunks [N, 2, Lk, Hkv, D]) in bf16, drawn as the module recipe says."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((cfg.lq, cfg.hq, cfg.d), generator=gen, dtype=torch.float32)
    kv = torch.randn((cfg.n_chunks, 2, cfg.lk, cfg.hkv, cfg.d), generator=gen, dtype=torch.float32)
    if cfg.qk_mult != 1.0:
        q.mul_(cfg.qk_mult)
        kv[:, 0].mul_(cfg.qk_mult)
    q = q.to(torch.bfloat16)
    kv = kv.to(torch.bfloat16)
    if device != "cpu":
        q = q.to(device)
        kv = kv.to(device)
    return q, kv


def to_f64(t: torch.Tensor):
    """Exact upcast of a (bf16) tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
