"""CPU checks of the comparison helpers the GPU parity tests use."""

import numpy as np

import oracle
from ring_inputs import RingConfig, make_inputs, to_f64
from tests.parity import compare, oracle_rows, wave_slice_rows


def test_per_kv_head_split_equals_one_call():
    cfg = RingConfig("split", rank=2, n_chunks=3, lq=96, lk=96, hq=6, hkv=3, d=64, causal=True)
    q, kv = make_inputs(cfg, seed=5)
    q64, kv64 = to_f64(q), to_f64(kv)
    rows = [0, 5, 31, 32, 64, 95]
    o1, l1 = oracle.ring_attention_rows(q64, kv64, cfg.rank, cfg.causal, cfg.gqa_ratio, rows)
    o2, l2 = oracle_rows(oracle, q64, kv64, cfg.rank, cfg.causal, cfg.gqa_ratio, rows, workers=3)
    assert np.abs(o1 - o2).max() <= 1e-13 and np.abs(l1 - l2).max() <= 1e-13


def test_wave_slice_rows_cover_every_slice():
    rows = wave_slice_rows(200, per_slice_random=1, seed=3)
    assert rows[0] == 0 and rows[-1] == 199
    assert {r // 32 for r in rows} == set(range(7))
    assert all(r in rows for r in (31, 32, 63, 64, 191, 192))


def test_strict_figures_reported():
    ref = np.array([[[1.0, 5.0]]])
    got = ref + np.array([[[0.009, 0.012]]])
    lref = np.array([[0.5]])
    rep = compare(got, lref + 6e-4, ref, lref)
    # 5.0 + 0.012 passes the widened bar (1e-2 + half a bf16 ulp of 5) but not plain 1e-2;
    # an lse of 0.5 off by 6e-4 passes the floored bar but is 1.2e-3 relative.
    assert rep["ok"] and rep["out_strict_over"] == 1
    assert abs(rep["lse_max_rel_err_strict"] - 1.2e-3) < 1e-12


def test_gemm_bar_accepts_rounding_and_rejects_a_wrong_term():
    from tests.parity import compare_gemm

    rng = np.random.default_rng(9)
    a = rng.standard_normal((8, 64))
    w = rng.standard_normal((16, 64))
    ref = a @ w.T
    abs_sum = np.abs(a) @ np.abs(w).T
    # the exact product rounded to bf16 passes
    rounded = np.array(ref, dtype=np.float32).view(np.uint32)
    rounded = ((rounded + 0x7FFF + ((rounded >> 16) & 1)) & 0xFFFF0000).view(np.float32).astype(np.float64)
    assert compare_gemm(rounded, ref, abs_sum, 64)["ok"]
    # dropping one k term does not
    wrong = a[:, :-1] @ w[:, :-1].T
    assert not compare_gemm(wrong, ref, abs_sum, 64)["ok"]


def test_gemm_bar_at_a_binade_boundary():
    """An exact value just below 2 whose fp32 sum lands past 2 + 2^-7 rounds to the bf16
    2 + 2^-6: the error is half an ulp of the upper binade plus the sum's error, which
    the bar allows; one ulp more is rejected."""
    from tests.parity import compare_gemm

    k = 64
    acc = (k / 16 + 16) * 2.0 ** -24
    abs_sum = np.array([[2 ** -7 / acc * 1.25]])   # accumulation bound 1.25 * 2^-7
    ref = np.array([[2.0 - 2.0 ** -9]])
    assert compare_gemm(np.array([[2.0 + 2.0 ** -6]]), ref, abs_sum, k)["ok"]
    assert not compare_gemm(np.array([[2.0 + 2.0 ** -5]]), ref, abs_sum, k)["ok"]
