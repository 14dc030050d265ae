"""Plain fp64 CPU oracles for the per-rank ring-attention forward and for one rank's
AllGather+GEMM.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (the HIP library and its Python binding) never imports it, and
this package never imports the product path: the two share no code.

Sources (the web pages on mKernel, cited by page title and section):
- "mKernel: multi-GPU, multi-node fused kernels" (project README), kernel table,
  Ring Attention row: per step, the local FlashAttention works on the KV chunk that
  arrived last while the next one moves around the ring.
- "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels" (arXiv 2609.13585), §4 and
  Table 3 (Ring Attention: sequence parallel; KV moved in tiles of 128 rows; no data
  dependency between compute and transfer inside one step), §3.2 and Eq. (2)
  (adaptive SM partition).
- The works that paper builds on, listed on its index page: FlashAttention-2 and
  "Ring Attention with Blockwise Transformers for Near-Infinite Context". The pages
  print no attention formula; the definition used here is the standard scaled
  dot-product softmax attention those works compute, written out in full.

- For AllGather+GEMM: the same paper, §4 and Table 3 (AllGather + GEMM row: shards
  moved in 128-row chunks, compute consumes them as they arrive, local shard first),
  and the README's kernel table (AllGather + GEMM row). The definition is the plain
  product of the gathered activation with the rank's weight shard.

Every function is pinned against brute force, closed forms and invariants
(``tests/test_oracle_pins.py``, ``tests/test_oracle_allgather_gemm.py``); none is
"parity unpinned".
"""

from .ring_attention import (  # noqa: F401
    ring_attention_reference,
    ring_attention_rows,
    ring_schedule,
    staging_tiles,
    controller_target,
    attention_flops,
)
from .allgather_gemm import (  # noqa: F401
    A_CHUNK_ROWS,
    allgather,
    allgather_gemm_reference,
    allgather_schedule,
    gemm_flops,
)
