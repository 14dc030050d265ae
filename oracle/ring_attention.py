"""fp64 CPU oracle: what one rank's ring-attention forward computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never calls
this module, and this module never calls the product path.

The method (mKernel paper "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", §4 and
Table 3, Ring Attention row; project README kernel table, Ring Attention row): a rank
holds one query chunk; KV chunks rotate around the ring; at each step the rank's local
FlashAttention consumes the chunk it holds, and its partial result is merged into the
accumulated output with the online softmax of FlashAttention-2 (running max, running
sum, log-sum-exp). That per-step merge is exact algebra (up to rounding), so the result
of all steps equals plain softmax attention of the rank's queries over the keys of the
whole concatenated sequence. This oracle computes that plain definition directly, in
float64, with no blocking over keys and no online merge.

Readings of points the pages leave open (each also listed in the design notes):
- softmax scale is 1/sqrt(D) (the FlashAttention convention);
- the log-sum-exp is the natural log of the sum of exp(scaled score), laid out [Hq, Lq];
- causal: chunks are contiguous, query i of rank r sits at global position r*L + i,
  key j of chunk c at c*L + j, and a query sees a key iff key_pos <= query_pos
  (so chunks after the rank are skipped and the diagonal chunk is lower-triangular,
  diagonal included);
- ring order: step t consumes chunk (rank - t) mod N (the local chunk first, then the
  chunk received from the predecessor); the result does not depend on it;
- grouped-query attention: query head h reads KV head floor(h / G).
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# Row granularity of a staged KV tile: Table 3 of the paper moves Ring Attention's KV in
# tiles of 128 rows.
KV_TILE_ROWS = 128


def ring_schedule(n_chunks: int, rank: int, causal: bool) -> List[int]:
    """Chunk consumed at each ring step, in step order.

    Step t (t = 0, 1, ...) consumes chunk (rank - t) mod n_chunks: step 0 is the rank's
    own chunk, which needs no transfer, and each later step the chunk that arrived from
    the predecessor (README kernel table, Ring Attention row: one KV chunk moves one hop
    around the ring per step). Under the causal reading, chunks after the rank hold only
    future keys and are skipped, so the rank runs rank+1 steps; otherwise it runs all
    n_chunks steps.
    """
    if n_chunks <= 0 or not (0 <= rank < n_chunks):
        raise ValueError("need 0 <= rank < n_chunks")
    n_steps = rank + 1 if causal else n_chunks
    return [(rank - t) % n_chunks for t in range(n_steps)]


def staging_tiles(lk: int, tile_rows: int = KV_TILE_ROWS) -> List[Tuple[int, int]]:
    """(first_row, n_rows) of each staged KV tile of a chunk of lk rows.

    Table 3 of the paper sets the transfer granularity of Ring Attention to KV tiles of
    128 rows; the last tile of a ragged chunk is short.
    """
    return [(r0, min(tile_rows, lk - r0)) for r0 in range(0, lk, tile_rows)]


def _check_shapes(q, kv, rank, causal, gqa_ratio):
    if q.ndim != 3 or kv.ndim != 5 or kv.shape[1] != 2:
        raise ValueError("q must be [Lq, Hq, D], kv_chunks [N, 2, Lk, Hkv, D]")
    lq, hq, d = q.shape
    n, _, lk, hkv, dk = kv.shape
    if dk != d:
        raise ValueError("head_dim mismatch")
    if gqa_ratio < 1 or hq != gqa_ratio * hkv:
        raise ValueError("need Hq == gqa_ratio * Hkv")
    if not (0 <= rank < n):
        raise ValueError("need 0 <= rank < n_chunks")
    if causal and lq != lk:
        raise ValueError("causal needs equal query and key chunk lengths")
    if lk == 0 and lq > 0:
        raise ValueError("no keys to attend to")
    return lq, hq, d, n, lk, hkv


def ring_attention_reference(
    q,
    kv_chunks,
    rank: int,
    causal: bool,
    gqa_ratio: int,
    query_rows: Optional[Sequence[int]] = None,
    block: int = 256,
) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of rank ``rank``'s queries over the full concatenated sequence.

    q:         [Lq, Hq, D]         query chunk of this rank (any real dtype; read as fp64)
    kv_chunks: [N, 2, Lk, Hkv, D]  all N chunks of the sequence, index 0 = K, 1 = V
    query_rows: optional subset of query indices (for sampled checks of large shapes)

    Returns (out, lse) in float64: out [n_rows, Hq, D], lse [Hq, n_rows], where
        s[i, p]  = <Q[i, h], K[p, g]> / sqrt(D),             g = h // gqa_ratio
        lse[h,i] = log( sum_{p valid for i} exp(s[i, p]) )
        out[i,h] = sum_{p valid for i} exp(s[i, p] - lse[h, i]) * V[p, g]
    summed over the keys p that query i may see (all keys, or key_pos <= query_pos
    under the causal reading). Keys a query may never see are not read at all, so
    non-finite values there cannot reach the result.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv_chunks, dtype=np.float64)
    lq, hq, d, n, lk, hkv = _check_shapes(q, kv, rank, causal, gqa_ratio)
    rows = np.arange(lq) if query_rows is None else np.asarray(query_rows, dtype=np.int64)

    # The concatenated sequence: key row p = c * Lk + j for chunk c, row j.
    keys = kv[:, 0].reshape(n * lk, hkv, d)
    vals = kv[:, 1].reshape(n * lk, hkv, d)
    scale = 1.0 / math.sqrt(d)

    out = np.empty((len(rows), hq, d), dtype=np.float64)
    lse = np.empty((hq, len(rows)), dtype=np.float64)
    for b0 in range(0, len(rows), block):
        r = rows[b0:b0 + block]
        if causal:
            qpos = rank * lq + r                       # global positions of the queries
            n_keys = int(qpos.max()) + 1               # keys beyond every query: unread
            visible = np.arange(n_keys)[None, :] <= qpos[:, None]
        else:
            n_keys = n * lk
            visible = np.ones((len(r), n_keys), dtype=bool)
        for h in range(hq):
            g = h // gqa_ratio
            s = (q[r, h, :] @ keys[:n_keys, g, :].T) * scale
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)                          # exp(-inf) = 0 for hidden keys
            z = e.sum(axis=1, keepdims=True)
            lse[h, b0:b0 + len(r)] = (m + np.log(z))[:, 0]
            out[b0:b0 + len(r), h, :] = (e @ vals[:n_keys, g, :]) / z
    return out, lse


def ring_attention_rows(q, kv_chunks, rank, causal, gqa_ratio, query_rows):
    """The same definition evaluated only at ``query_rows`` (sampled full-size checks)."""
    return ring_attention_reference(q, kv_chunks, rank, causal, gqa_ratio, query_rows=query_rows)


def attention_flops(lq: int, lk: int, n_chunks: int, rank: int, causal: bool, hq: int, d: int) -> int:
    """Algorithmic FLOPs of the forward: 4 * D * Hq * (number of visible (query, key) pairs).

    Each visible pair costs one D-long dot product for the score and one D-long
    multiply-add into the output: 2*D + 2*D FLOPs. Masked pairs and skipped chunks are
    not counted (exact triangle, not half of the full square).
    """
    if causal:
        # r full chunks before the diagonal, then a lower triangle with the diagonal.
        pairs = rank * lq * lk + lq * (lq + 1) // 2
    else:
        pairs = n_chunks * lq * lk
    return 4 * d * hq * pairs


def controller_target(b: int, r_p: int, r_s: int, c_p: float, c_s: float) -> float:
    """Eq. (2) of the paper (§3.2): the staging-role block count that equalizes the
    predicted completion times of the two roles.

    b: blocks in the grid; r_p, r_s: remaining compute / staging tasks; c_p, c_s: their
    estimated per-task costs. The compute role then needs r_p*c_p/(b - n) and the
    staging role r_s*c_s/n; setting the two equal and solving for n gives
    n = b * r_s*c_s / (r_p*c_p + r_s*c_s). Returns the real-valued n (the kernel's
    integer rounding and clamping are its own, documented where it implements them).
    """
    work_s = float(r_s) * float(c_s)
    work_p = float(r_p) * float(c_p)
    if work_s + work_p == 0.0:
        return 0.0
    return b * work_s / (work_p + work_s)
