"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each check takes an oracle function with the signature of
``oracle.ring_attention_reference`` and raises AssertionError when it disagrees with
what the definition (scaled dot-product softmax attention over the concatenated ring
sequence; mKernel paper §4 / Table 3 Ring Attention, via FlashAttention-2 and Ring
Attention) fixes:

  P0  hand-worked closed forms stored in tests/golden/hand_worked.json
  P1  brute force with scalar loops on tiny inputs, causal visibility phrased per chunk
  P2  per-chunk softmax + log-sum-exp merge (scipy) in ring order and in random orders
  P3  constant V rows return that row
  P4  a single key returns its value; lse is its scaled score
  P5  causal: non-finite values in chunks after the rank do not change the result
  P6  Q = 0: lse = ln(number of visible keys), out = mean of the visible V rows
  P7  grouped-query attention equals MHA on repeat-interleaved KV heads
  P8  non-causal: the result does not depend on the rank
  P9  translating every key by a vector a leaves out unchanged and shifts lse by <q,a>/sqrt(D)

The mutation tests at the end plant plausible mistakes in copies of the oracle source
and require that at least one of these checks fails for each of them.
"""

import json
import math
import os
import random
import types

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from oracle import ring_attention as oracle_mod

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _rand_case(rng, n, l, hkv, g, d, scale=1.0):
    q = rng.standard_normal((l, hkv * g, d)) * scale
    kv = rng.standard_normal((n, 2, l, hkv, d)) * scale
    return q, kv


# ----------------------------------------------------------------------------- checks

def check_hand_worked(fn):
    doc = json.load(open(GOLDEN))
    for case in doc["cases"]:
        out, lse = fn(np.array(case["q"], float), np.array(case["kv"], float), case["rank"], case["causal"],
                      case["gqa_ratio"])
        np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(lse, np.array(case["lse"]), rtol=0, atol=1e-14, err_msg=case["name"])


def _brute(q, kv, rank, causal, g):
    """Scalar loops; visibility phrased per chunk: earlier chunks fully visible, the
    rank's own chunk lower-triangular with the diagonal, later chunks hidden."""
    lq, hq, d = q.shape
    n, _, lk, hkv, _ = kv.shape
    out = np.zeros((lq, hq, d))
    lse = np.zeros((hq, lq))
    for h in range(hq):
        kvh = h // g
        for i in range(lq):
            scores, values = [], []
            for c in range(n):
                for j in range(lk):
                    if causal and (c > rank or (c == rank and j > i)):
                        continue
                    dot = 0.0
                    for x in range(d):
                        dot += q[i, h, x] * kv[c, 0, j, kvh, x]
                    scores.append(dot / math.sqrt(d))
                    values.append(kv[c, 1, j, kvh, :])
            z = sum(math.exp(s) for s in scores)
            lse[h, i] = math.log(z)
            for s, v in zip(scores, values):
                out[i, h, :] += math.exp(s) / z * v
    return out, lse


def check_bruteforce(fn):
    rng = np.random.default_rng(1)
    for (n, l, hkv, g, d) in [(1, 1, 1, 1, 1), (2, 3, 1, 2, 4), (4, 4, 2, 1, 3), (3, 2, 1, 2, 2), (4, 3, 2, 2, 4)]:
        q, kv = _rand_case(rng, n, l, hkv, g, d)
        for causal in (False, True):
            for rank in range(n):
                out, lse = fn(q, kv, rank, causal, g)
                bo, bl = _brute(q, kv, rank, causal, g)
                np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def _chunk_partial(q, kv_c, g, mask=None):
    """out and lse of one head group against one chunk alone (scipy softmax/logsumexp)."""
    lq, hq, d = q.shape
    o = np.zeros((lq, hq, d))
    l_ = np.full((hq, lq), -np.inf)
    for h in range(hq):
        s = q[:, h, :] @ kv_c[0, :, h // g, :].T / math.sqrt(d)
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        ok = np.isfinite(s).any(axis=1)
        w = np.zeros_like(s)
        w[ok] = softmax(s[ok], axis=1)
        o[:, h, :] = w @ kv_c[1, :, h // g, :]
        l_[h, ok] = logsumexp(s[ok], axis=1)
    return o, l_


def _merge(parts):
    o_acc, l_acc = parts[0]
    for o, l_ in parts[1:]:
        l_new = np.logaddexp(l_acc, l_)
        wa = np.exp(l_acc - l_new).T[:, :, None]
        wb = np.exp(l_ - l_new).T[:, :, None]
        o_acc = np.nan_to_num(wa) * o_acc + np.nan_to_num(wb) * o
        l_acc = l_new
    return o_acc, l_acc


def check_chunk_merge(fn):
    rng = np.random.default_rng(2)
    n, l, hkv, g, d = 5, 6, 2, 2, 8
    q, kv = _rand_case(rng, n, l, hkv, g, d)
    for causal in (False, True):
        for rank in (0, 2, 4):
            steps = [(rank - t) % n for t in range(rank + 1 if causal else n)]
            parts = {}
            for c in steps:
                mask = None
                if causal and c == rank:
                    mask = np.arange(l)[None, :] <= np.arange(l)[:, None]
                parts[c] = _chunk_partial(q, kv[c], g, mask)
            out, lse = fn(q, kv, rank, causal, g)
            orders = [steps] + [random.Random(k).sample(steps, len(steps)) for k in range(3)]
            for order in orders:
                mo, ml = _merge([parts[c] for c in order])
                np.testing.assert_allclose(out, mo, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse, ml, rtol=0, atol=1e-12)


def check_constant_v(fn):
    rng = np.random.default_rng(3)
    n, l, hkv, g, d = 3, 7, 2, 2, 16
    q, kv = _rand_case(rng, n, l, hkv, g, d, scale=3.0)
    u = rng.standard_normal((hkv, d))
    kv[:, 1] = u[None, None, :, :]
    for causal in (False, True):
        out, _ = fn(q, kv, 1, causal, g)
        for h in range(hkv * g):
            np.testing.assert_allclose(out[:, h, :], np.broadcast_to(u[h // g], (l, d)), rtol=0, atol=1e-12)


def check_single_key(fn):
    rng = np.random.default_rng(4)
    d = 8
    q = rng.standard_normal((1, 1, d))
    kv = rng.standard_normal((1, 2, 1, 1, d))
    for causal in (False, True):
        out, lse = fn(q, kv, 0, causal, 1)
        np.testing.assert_allclose(out[0, 0], kv[0, 1, 0, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], float(q[0, 0] @ kv[0, 0, 0, 0]) / math.sqrt(d), rtol=0, atol=1e-14)
    # Causal rank 0, row 0 of any shape sees key 0 only.
    q, kv = _rand_case(rng, 4, 5, 2, 2, d)
    out, lse = fn(q, kv, 0, True, 2)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], kv[0, 1, 0, h // 2], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[h, 0], float(q[0, h] @ kv[0, 0, 0, h // 2]) / math.sqrt(d), rtol=0,
                                   atol=1e-13)


def check_future_chunks_unread(fn):
    rng = np.random.default_rng(5)
    n, l, hkv, g, d = 5, 4, 1, 2, 8
    q, kv = _rand_case(rng, n, l, hkv, g, d)
    for rank in range(n):
        ref_o, ref_l = fn(q, kv, rank, True, g)
        bad = kv.copy()
        bad[rank + 1:] = np.nan
        bad_o, bad_l = fn(q, bad, rank, True, g)
        assert np.array_equal(ref_o, bad_o) and np.array_equal(ref_l, bad_l)
        noisy = kv.copy()
        noisy[rank + 1:] = 1e3 * rng.standard_normal(noisy[rank + 1:].shape)
        n_o, n_l = fn(q, noisy, rank, True, g)
        assert np.array_equal(ref_o, n_o) and np.array_equal(ref_l, n_l)


def check_zero_q(fn):
    rng = np.random.default_rng(6)
    n, l, hkv, g, d = 4, 6, 2, 1, 4
    _, kv = _rand_case(rng, n, l, hkv, g, d)
    q = np.zeros((l, hkv * g, d))
    vals = kv[:, 1].reshape(n * l, hkv, d)
    for causal in (False, True):
        for rank in (0, 3):
            out, lse = fn(q, kv, rank, causal, g)
            for i in range(l):
                nvis = rank * l + i + 1 if causal else n * l
                np.testing.assert_allclose(lse[:, i], math.log(nvis), rtol=0, atol=1e-13)
                for h in range(hkv * g):
                    np.testing.assert_allclose(out[i, h], vals[:nvis, h // g].mean(axis=0), rtol=0, atol=1e-13)


def check_gqa_is_repeated_mha(fn):
    rng = np.random.default_rng(7)
    n, l, hkv, g, d = 3, 5, 2, 4, 8
    q, kv = _rand_case(rng, n, l, hkv, g, d)
    rep = np.repeat(kv, g, axis=3)  # KV head k -> query heads k*g .. k*g+g-1
    for causal in (False, True):
        o1, l1 = fn(q, kv, 2, causal, g)
        o2, l2 = fn(q, rep, 2, causal, 1)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def check_noncausal_rank_invariance(fn):
    rng = np.random.default_rng(8)
    q, kv = _rand_case(rng, 4, 3, 1, 2, 4)
    o0, l0 = fn(q, kv, 0, False, 2)
    for r in (1, 2, 3):
        o, l_ = fn(q, kv, r, False, 2)
        np.testing.assert_allclose(o, o0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l_, l0, rtol=0, atol=1e-13)


def check_key_translation(fn):
    rng = np.random.default_rng(9)
    n, l, hkv, g, d = 3, 4, 2, 2, 8
    q, kv = _rand_case(rng, n, l, hkv, g, d)
    for mag in (1.0, 3000.0):  # the second shifts scores by thousands: exp must not overflow
        a = rng.standard_normal((hkv, d))
        a *= mag / np.abs(a).max()
        moved = kv.copy()
        moved[:, 0] += a[None, None, :, :]
        for causal in (False, True):
            o1, l1 = fn(q, kv, 1, causal, g)
            o2, l2 = fn(q, moved, 1, causal, g)
            shift = np.einsum("ihd,hd->hi", q, np.repeat(a, g, axis=0)) / math.sqrt(d)
            np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-9 * mag)
            np.testing.assert_allclose(l2, l1 + shift, rtol=0, atol=1e-11 * mag)


PIN_CHECKS = [
    check_hand_worked,
    check_bruteforce,
    check_chunk_merge,
    check_constant_v,
    check_single_key,
    check_future_chunks_unread,
    check_zero_q,
    check_gqa_is_repeated_mha,
    check_noncausal_rank_invariance,
    check_key_translation,
]


@pytest.mark.parametrize("check", PIN_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.ring_attention_reference)


def test_query_row_subset_matches_full():
    rng = np.random.default_rng(10)
    q, kv = _rand_case(rng, 3, 9, 2, 2, 8)
    for causal in (False, True):
        fo, fl = oracle.ring_attention_reference(q, kv, 2, causal, 2, block=4)
        rows = [0, 3, 8, 5]
        so, sl = oracle.ring_attention_rows(q, kv, 2, causal, 2, rows)
        np.testing.assert_allclose(so, fo[rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(sl, fl[:, rows], rtol=0, atol=1e-13)


# ------------------------------------------------------------------- other oracle pins

def test_ring_schedule_properties():
    for n in range(1, 9):
        for rank in range(n):
            nc = oracle.ring_schedule(n, rank, False)
            assert nc[0] == rank and sorted(nc) == list(range(n))
            for a, b in zip(nc, nc[1:]):
                assert b == (a - 1) % n  # each step brings the predecessor's chunk
            c = oracle.ring_schedule(n, rank, True)
            assert c == nc[:rank + 1] and sorted(c) == list(range(rank + 1))


def test_staging_tiles_cover_chunk():
    for lk in (1, 127, 128, 129, 1000, 4096):
        tiles = oracle.staging_tiles(lk)
        assert tiles[0][0] == 0 and sum(n for _, n in tiles) == lk
        for (a, na), (b, _) in zip(tiles, tiles[1:]):
            assert b == a + na and na == 128
        assert 0 < tiles[-1][1] <= 128


def test_attention_flops_counts_visible_pairs():
    for (n, l, rank, causal) in [(4, 5, 0, False), (4, 5, 2, True), (3, 7, 2, True), (1, 3, 0, True)]:
        vis = 0
        for i in range(l):
            for c in range(n):
                for j in range(l):
                    if not causal or c * l + j <= rank * l + i:
                        vis += 1
        assert oracle.attention_flops(l, l, n, rank, causal, 3, 16) == 4 * 16 * 3 * vis


def test_controller_target_equalizes_completion_times():
    rng = random.Random(11)
    for _ in range(200):
        b = rng.randint(2, 512)
        rp, rs = rng.randint(1, 10000), rng.randint(1, 10000)
        cp, cs = rng.uniform(1, 1e6), rng.uniform(1, 1e6)
        n = oracle.controller_target(b, rp, rs, cp, cs)
        assert 0 < n < b
        # Predicted completion of each role with its share of the blocks (paper §3.2).
        assert math.isclose(rs * cs / n, rp * cp / (b - n), rel_tol=1e-9)
    assert oracle.controller_target(64, 100, 0, 5.0, 7.0) == 0.0
    assert oracle.controller_target(64, 0, 100, 5.0, 7.0) == 64.0
    assert oracle.controller_target(64, 10, 10, 3.0, 3.0) == 32.0


# ---------------------------------------------------------------- planted mistakes

MUTATIONS = {
    "scale_1_over_d": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "strict_causal": ("np.arange(n_keys)[None, :] <= qpos[:, None]", "np.arange(n_keys)[None, :] < qpos[:, None]"),
    "causal_no_rank_offset": ("qpos = rank * lq + r ", "qpos = r "),
    "gqa_modulo": ("g = h // gqa_ratio\n            s = (q", "g = h % hkv\n            s = (q"),
    "lse_dropped_max": ("(m + np.log(z))[:, 0]", "np.log(z)[:, 0]"),
    "unnormalized_out": ("(e @ vals[:n_keys, g, :]) / z", "(e @ vals[:n_keys, g, :])"),
    "k_v_swapped": ("keys = kv[:, 0].reshape", "keys = kv[:, 1].reshape"),
    "scores_use_values": ("@ keys[:n_keys, g, :].T", "@ vals[:n_keys, g, :].T"),
    "chunk_row_order": ("keys = kv[:, 0].reshape(n * lk, hkv, d)",
                        "keys = kv[:, 0].transpose(1, 0, 2, 3).reshape(n * lk, hkv, d)"),
    "no_max_subtraction_in_lse": ("e = np.exp(s - m)", "e = np.exp(s); m = 0 * m"),
    "sum_over_hidden_keys": ("s = np.where(visible, s, -np.inf)", "s = s"),
}


def _mutant(src_from, src_to):
    src = open(oracle_mod.__file__).read()
    assert src.count(src_from) == 1, src_from
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(src_from, src_to), "oracle_mutant", "exec"), mod.__dict__)
    return mod.ring_attention_reference


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    fn = _mutant(*MUTATIONS[name])
    failed = []
    for check in PIN_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(fn)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
