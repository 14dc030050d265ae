"""Writes hand_worked.json: hand-derived closed forms of softmax attention.

Each case's numbers follow from the derivation text stored beside them and are
evaluated with Python's math module only; nothing here calls the oracle or the HIP
path. Run from the repository root: python tests/golden/make_hand_worked.py
"""
import json
import math
import os

e = math.e
cases = []
A = dict(
    name="two_keys_noncausal",
    derivation=("D=4, scale=1/2. One query q=[2,0,0,0]; chunk 0 holds K=[1,0,0,0], V=[1,0,0,0]; chunk 1 holds "
                "K=[0,0,0,0], V=[0,1,0,0]. Scores: 2*1/2 = 1 and 0. lse = ln(e+1). Weights e/(e+1), 1/(e+1), "
                "so out = [e/(e+1), 1/(e+1), 0, 0]."),
    rank=0, causal=False, gqa_ratio=1,
    q=[[[2, 0, 0, 0]]],
    kv=[[[[[1, 0, 0, 0]]], [[[1, 0, 0, 0]]]], [[[[0, 0, 0, 0]]], [[[0, 1, 0, 0]]]]],
    out=[[[e / (e + 1), 1 / (e + 1), 0.0, 0.0]]],
    lse=[[math.log(e + 1)]],
)
cases.append(A)
z1 = 2 * e + 1 + math.exp(-2)
cases.append(dict(
    name="causal_rank1_of2_L2",
    derivation=("D=4, scale=1/2, chunks of L=2, rank 1 of 2, causal. Key positions: chunk 0 -> 0,1; chunk 1 -> 2,3. "
                "Query 0 of rank 1 sits at position 2 and sees keys 0..2; query 1 at position 3 sees keys 0..3. "
                "K rows: [1,0,0,0],[0,1,0,0],[0,0,1,0],[-1,-1,0,0]; V rows: unit vectors e0..e3. "
                "Query 0 = 0: all three scores 0, lse = ln 3, out = [1/3,1/3,1/3,0]. "
                "Query 1 = [2,2,0,0]: scores 1, 1, 0, -2; Z = 2e + 1 + e^-2; lse = ln Z; "
                "out = [e, e, 1, e^-2] / Z."),
    rank=1, causal=True, gqa_ratio=1,
    q=[[[0, 0, 0, 0]], [[2, 2, 0, 0]]],
    kv=[[[[[1, 0, 0, 0]], [[0, 1, 0, 0]]], [[[1, 0, 0, 0]], [[0, 1, 0, 0]]]],
        [[[[0, 0, 1, 0]], [[-1, -1, 0, 0]]], [[[0, 0, 1, 0]], [[0, 0, 0, 1]]]]],
    out=[[[1 / 3, 1 / 3, 1 / 3, 0.0]], [[e / z1, e / z1, 1 / z1, math.exp(-2) / z1]]],
    lse=[[math.log(3), math.log(z1)]],
))
cases.append(dict(
    name="gqa2_one_kv_head",
    derivation=("Case two_keys_noncausal's KV, one KV head shared by two query heads (G=2). Head 0 query "
                "[2,0,0,0] gives that case's result; head 1 query 0 gives equal weights: out = [1/2,1/2,0,0], "
                "lse = ln 2."),
    rank=0, causal=False, gqa_ratio=2,
    q=[[[2, 0, 0, 0], [0, 0, 0, 0]]],
    kv=A["kv"],
    out=[[[e / (e + 1), 1 / (e + 1), 0.0, 0.0], [0.5, 0.5, 0.0, 0.0]]],
    lse=[[math.log(e + 1)], [math.log(2)]],
))
doc = {
    "source": ("Hand-worked closed forms of scaled dot-product softmax attention, the computation the mKernel "
               "paper's Ring Attention kernel performs per rank (paper 'mKernel: Fast Multi-GPU, Multi-Node Fused "
               "Kernels', Section 4, Table 3; definition from the FlashAttention-2 and Ring Attention works it "
               "builds on). The pages print no worked numbers, so each value here is derived by hand in "
               "'derivation' and evaluated with Python's math module."),
    "layout": "q [Lq, Hq, D]; kv [N, 2, Lk, Hkv, D] (index 0 = K, 1 = V); out [Lq, Hq, D]; lse [Hq, Lq]",
    "cases": cases,
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_worked.json"), "w") as f:
    json.dump(doc, f, indent=1)
