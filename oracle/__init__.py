"""Plain fp64 CPU oracle for the per-rank ring-attention forward.

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

Every function is pinned by ``tests/test_oracle_pins.py`` against brute force,
closed forms and invariants; none is "parity unpinned".
"""

from .ring_attention import (  # noqa: F401
    ring_attention_reference,
    ring_attention_rows,
    ring_schedule,
    staging_tiles,
    controller_target,
    attention_flops,
)
