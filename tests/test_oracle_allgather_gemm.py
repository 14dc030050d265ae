"""Pins of the AllGather+GEMM oracle to facts that do not come from the oracle itself
(mKernel paper §4 and Table 3, AllGather + GEMM row; README kernel table):

  G0  hand-worked cases in tests/golden/ag_gemm_hand_worked.json (transpose convention,
      shard placement)
  G1  scalar brute force on tiny inputs
  G2  W = identity returns the gathered activation
  G3  shard r filled with r+1 and W = ones: row i of C is (shard of i + 1) * K
  G4  the rows of shard r in C equal that shard's own product with W^T (a library
      matmul of the shard alone, no concatenation)
  G5  the result does not depend on the rank; the schedule is a permutation that
      starts with the local shard and then walks the ring backwards

Mutations planted in copies of the oracle source must each fail at least one pin.
"""

import json
import os
import types

import numpy as np
import pytest

import oracle
from oracle import allgather_gemm as ag_mod

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ag_gemm_hand_worked.json")


def check_hand_worked(fn):
    for case in json.load(open(GOLDEN))["cases"]:
        a_full, c = fn(np.array(case["a_shards"], float), np.array(case["w"], float), case["rank"])
        np.testing.assert_array_equal(a_full, np.array(case["a_full"], float), err_msg=case["name"])
        np.testing.assert_array_equal(c, np.array(case["c"], float), err_msg=case["name"])


def check_brute(fn):
    rng = np.random.default_rng(3)
    for n, m, k, no in ((1, 1, 1, 1), (2, 3, 4, 5), (4, 2, 3, 2)):
        a = rng.standard_normal((n, m, k))
        w = rng.standard_normal((no, k))
        a_full, c = fn(a, w, n - 1)
        for r in range(n):
            for i in range(m):
                for j in range(no):
                    s = 0.0
                    for t in range(k):
                        s += a[r, i, t] * w[j, t]
                    assert abs(c[r * m + i, j] - s) <= 1e-12
                    assert all(a_full[r * m + i, t] == a[r, i, t] for t in range(k))


def check_identity(fn):
    rng = np.random.default_rng(4)
    a = rng.standard_normal((3, 5, 7))
    _, c = fn(a, np.eye(7), 2)
    np.testing.assert_array_equal(c, a.reshape(15, 7))


def check_shard_placement(fn):
    n, m, k = 4, 3, 6
    a = np.stack([np.full((m, k), r + 1.0) for r in range(n)])
    _, c = fn(a, np.ones((2, k)), 1)
    for i in range(n * m):
        assert c[i, 0] == c[i, 1] == (i // m + 1) * k


def check_per_shard(fn):
    rng = np.random.default_rng(5)
    a = rng.standard_normal((3, 4, 8))
    w = rng.standard_normal((6, 8))
    _, c = fn(a, w, 0)
    for r in range(3):
        np.testing.assert_allclose(c[r * 4:(r + 1) * 4], np.matmul(a[r], w.T), rtol=0, atol=1e-12)


def check_rank_and_schedule(fn, sched):
    rng = np.random.default_rng(6)
    a = rng.standard_normal((5, 2, 3))
    w = rng.standard_normal((4, 3))
    ref = fn(a, w, 0)[1]
    for r in range(5):
        np.testing.assert_array_equal(fn(a, w, r)[1], ref)
        s = sched(5, r)
        assert s[0] == r and sorted(s) == list(range(5))
        assert all(s[i + 1] == (s[i] - 1) % 5 for i in range(4))


CHECKS = [check_hand_worked, check_brute, check_identity, check_shard_placement, check_per_shard]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_pins(check):
    check(oracle.allgather_gemm_reference)


def test_schedule_and_rank_invariance():
    check_rank_and_schedule(oracle.allgather_gemm_reference, oracle.allgather_schedule)


def test_flops():
    assert oracle.gemm_flops(16384, 4096, 8192) == 2 * 16384 * 4096 * 8192


MUTATIONS = [
    ("weight not transposed", "return a_full, a_full @ w.T", "return a_full, a_full @ w"),
    ("shards gathered in reverse", "return a.reshape(n * m_loc, k)", "return a[::-1].reshape(n * m_loc, k)"),
    ("local shard first in A_full", "a_full = allgather(a)",
     "a_full = allgather(np.concatenate([a[rank:rank + 1], np.delete(a, rank, axis=0)]))"),
    ("rows of a shard transposed in place", "return a.reshape(n * m_loc, k)",
     "return a.transpose(1, 0, 2).reshape(n * m_loc, k)"),
    ("schedule walks forward", "return [(rank - i) % n_ranks for i in range(n_ranks)]",
     "return [(rank + i) % n_ranks for i in range(n_ranks)]"),
    ("output scaled by the shard count", "return a_full, a_full @ w.T", "return a_full, (a_full @ w.T) * a.shape[0]"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mutations_are_caught(name, old, new):
    src = open(ag_mod.__file__).read()
    assert old in src, name
    mod = types.ModuleType("ag_mutant")
    exec(compile(src.replace(old, new, 1), "ag_mutant", "exec"), mod.__dict__)
    caught = False
    for check in CHECKS:
        try:
            check(mod.allgather_gemm_reference)
        except (AssertionError, ValueError, IndexError):
            caught = True
            break
    if not caught:
        try:
            check_rank_and_schedule(mod.allgather_gemm_reference, mod.allgather_schedule)
        except (AssertionError, ValueError, IndexError):
            caught = True
    assert caught, f"mutation '{name}' passed every pin"
