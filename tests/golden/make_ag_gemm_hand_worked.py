"""Writes ag_gemm_hand_worked.json: hand-derived AllGather+GEMM cases.

Each case's expected matrices follow from the derivation text beside them, written out
by hand here (plain Python lists, no numerical library); nothing calls the oracle or the
HIP path. Run from the repository root: python tests/golden/make_ag_gemm_hand_worked.py
"""
import json
import os

cases = [
    dict(
        name="two_ranks_transpose_convention",
        derivation=("N=2 ranks, M_loc=1, K=2, N_out=2, rank 1. Shards: rank 0 holds [[1, 2]], rank 1 holds "
                    "[[3, 4]]. Gathered A_full = [[1, 2], [3, 4]] (shard 0 first, whatever the rank). "
                    "W = [[1, 0], [1, 1]] is [N_out, K]; C = A_full W^T: row [1,2] -> [1*1+2*0, 1*1+2*1] = [1, 3]; "
                    "row [3,4] -> [3, 7]. (A_full W would give [[3, 2], [7, 4]].)"),
        rank=1,
        a_shards=[[[1, 2]], [[3, 4]]],
        w=[[1, 0], [1, 1]],
        a_full=[[1, 2], [3, 4]],
        c=[[1, 3], [3, 7]],
    ),
    dict(
        name="three_ranks_two_rows_each",
        derivation=("N=3, M_loc=2, K=3, N_out=1, rank 0. Shard r holds rows [r, 1, 0] and [0, r, 1]. "
                    "A_full rows in shard order: [0,1,0],[0,0,1],[1,1,0],[0,1,1],[2,1,0],[0,2,1]. "
                    "W = [[1, 10, 100]]: C = [1*a0 + 10*a1 + 100*a2] per row = 10, 100, 11, 110, 12, 120."),
        rank=0,
        a_shards=[[[0, 1, 0], [0, 0, 1]], [[1, 1, 0], [0, 1, 1]], [[2, 1, 0], [0, 2, 1]]],
        w=[[1, 10, 100]],
        a_full=[[0, 1, 0], [0, 0, 1], [1, 1, 0], [0, 1, 1], [2, 1, 0], [0, 2, 1]],
        c=[[10], [100], [11], [110], [12], [120]],
    ),
]
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ag_gemm_hand_worked.json")
with open(path, "w") as f:
    json.dump({"source": "hand-derived (tests/golden/make_ag_gemm_hand_worked.py)", "cases": cases}, f, indent=1)
    f.write("\n")
print(path)
