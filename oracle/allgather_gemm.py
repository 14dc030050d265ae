"""fp64 CPU oracle: what one rank's AllGather+GEMM computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never calls
this module, and this module never calls the product path.

The method (mKernel paper "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", §4 and
Table 3, AllGather + GEMM row; project README kernel table, AllGather + GEMM row):
each of the N ranks of a tensor-parallel group holds a shard of the activation A
(a block of rows); the ranks gather every shard (AllGather) and each rank multiplies
the gathered A by its own weight shard. In the fused kernel the GEMM consumes the
gathered rows as they arrive, in 128-row chunks (Table 3), the local shard first
(§4: compute tiles are ordered by input availability). The result does not depend on
that order: it is the plain product of the gathered matrix with the weight shard,
which this oracle computes directly in float64.

Readings of points the pages leave open (each also listed in the design notes):
- layout: shards a_shards[r] are [M_loc, K], row-major; the gathered A_full is
  [N * M_loc, K] with shard r at rows r*M_loc .. (r+1)*M_loc - 1;
- the weight shard is given as W [N_out, K] (the layout of a linear layer's weight)
  and the GEMM is C = A_full @ W^T, [N * M_loc, N_out];
- shard order consumed by rank r: its own shard first, then (r - 1) mod N,
  (r - 2) mod N, ... (received from the ring predecessor); the result does not
  depend on it.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np

# Row granularity of a gathered A chunk: Table 3 of the paper moves AllGather+GEMM's
# shards in chunks of 128 rows.
A_CHUNK_ROWS = 128


def allgather_schedule(n_ranks: int, rank: int) -> List[int]:
    """Shards in the order rank `rank` consumes them: its own first (§4: the local
    shard is processed first), then the shards received from the ring predecessor."""
    if n_ranks <= 0 or not (0 <= rank < n_ranks):
        raise ValueError("need 0 <= rank < n_ranks")
    return [(rank - i) % n_ranks for i in range(n_ranks)]


def allgather(a_shards) -> np.ndarray:
    """The gathered activation: shard r at rows r*M_loc .. (r+1)*M_loc - 1."""
    a = np.asarray(a_shards, dtype=np.float64)
    if a.ndim != 3:
        raise ValueError("a_shards must be [N, M_loc, K]")
    n, m_loc, k = a.shape
    return a.reshape(n * m_loc, k)


def allgather_gemm_reference(a_shards, w, rank: int) -> Tuple[np.ndarray, np.ndarray]:
    """(A_full, C) of one rank's AllGather+GEMM, in float64.

    a_shards: [N, M_loc, K]  every rank's activation shard (read as fp64)
    w:        [N_out, K]     this rank's weight shard
    rank:     0 <= rank < N  (the result does not depend on it; it is checked)
    Returns A_full [N*M_loc, K] and C = A_full @ W^T [N*M_loc, N_out].
    """
    a = np.asarray(a_shards, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if a.ndim != 3 or w.ndim != 2 or w.shape[1] != a.shape[2]:
        raise ValueError("a_shards [N, M_loc, K], w [N_out, K]")
    allgather_schedule(a.shape[0], rank)  # validates the rank
    a_full = allgather(a)
    return a_full, a_full @ w.T


def gemm_flops(m: int, n: int, k: int) -> int:
    """Algorithmic FLOPs of an m x n x k product: one multiply and one add per term."""
    return 2 * m * n * k
