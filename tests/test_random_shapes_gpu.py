"""Seeded random small shapes and launch options against the fp64 oracles (HIP path,
through the C ABI). Ring attention: ragged lengths, any KV-head count and GQA ratio,
both head sizes, causal or not, with random staging pieces, task sizes, step modes,
splits and grids. AllGather+GEMM: any rank count and shard height, K and N_out over
their supported multiples, random splits and grids. Every case prints what it runs
before launching."""

import numpy as np
import pytest
import torch

import oracle
import overlap_attention_amd as mk
from ag_inputs import AgConfig, make_ag_inputs
from ring_inputs import RingConfig, make_inputs, to_f64
from tests.parity import compare, compare_gemm, fmt

pytestmark = pytest.mark.gpu

N_CASES = 64
N_AG_CASES = 24


def random_case(i):
    r = np.random.default_rng(1000 + i)
    n = int(r.integers(1, 11))
    rank = int(r.integers(0, n))
    causal = bool(r.integers(0, 2))
    hkv = int(r.integers(1, 7))
    gqa = int(r.choice([1, 2, 3, 4, 8]))
    d = int(r.choice([64, 128]))
    lq = int(r.integers(1, 321))
    lk = lq if causal else int(r.integers(1, 321))
    cfg = RingConfig(f"rand{i}_r{rank}of{n}_q{lq}_k{lk}_h{hkv * gqa}kv{hkv}_d{d}_{'c' if causal else 'nc'}",
                     rank=rank, n_chunks=n, lq=lq, lk=lk, hq=hkv * gqa, hkv=hkv, d=d, causal=causal)
    kw = dict(spin_timeout_us=5_000_000,
              stage_pieces=int(r.choice([0, 1, 2, 3, hkv])),
              steps_per_task=int(r.integers(0, 5)),
              parallel_steps=int(r.choice([-1, 0, 1])),
              grid_wgs=int(r.choice([0, 1, 3, 7, 16])))
    split = int(r.integers(0, 3))
    kw["split_mode"] = split
    if split == mk.MK_SPLIT_FIXED:
        kw["fixed_staging_wgs"] = int(r.integers(0, 4))
    if r.integers(0, 4) == 0:
        kw["stage_delay_ticks"] = 2000
    return cfg, kw


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    cfg, kw = random_case(i)
    print(f"[case] {cfg} opts={kw}", flush=True)
    q, kv = make_inputs(cfg, seed=i)
    out, lse, st = mk.ring_attn_fwd(q.cuda(), kv.cuda(), cfg.rank, cfg.causal, cfg.gqa_ratio,
                                    opts=mk.default_opts(**kw), want_stats=True)
    mk.mk_ring_attn_status()
    print("    stats:", {k: st[k] for k in ("grid_wgs", "n_steps", "step_groups", "parallel_steps", "stage_pieces",
                                              "n_stage_tasks", "staging_tasks_done", "compute_tasks_done")}, flush=True)
    assert st["status"] == 0
    assert st["staging_tasks_done"] == st["n_stage_tasks"]
    assert st["compute_tasks_done"] == st["n_units"] * st["n_steps"]
    ref_o, ref_l = oracle.ring_attention_reference(to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio)
    rep = compare(to_f64(out), lse.double().cpu().numpy(), ref_o, ref_l)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


def random_ag_case(i):
    r = np.random.default_rng(5000 + i)
    n = int(r.integers(1, 9))
    rank = int(r.integers(0, n))
    m_loc = int(r.integers(1, 400))
    k = 64 * int(r.integers(1, 9))
    n_out = 8 * int(r.integers(1, 129))
    cfg = AgConfig(f"ag_rand{i}_r{rank}of{n}_M{m_loc}_K{k}_N{n_out}", n_ranks=n, rank=rank, m_loc=m_loc, k=k,
                   n_out=n_out)
    kw = dict(spin_timeout_us=5_000_000, grid_wgs=int(r.choice([0, 1, 3, 7, 16])))
    split = int(r.integers(0, 3))
    kw["split_mode"] = split
    if split == mk.MK_SPLIT_FIXED:
        kw["fixed_staging_wgs"] = int(r.integers(0, 4))
    return cfg, kw


@pytest.mark.parametrize("i", range(N_AG_CASES))
def test_random_allgather_gemm_matches_oracle(i):
    cfg, kw = random_ag_case(i)
    print(f"[case] {cfg} opts={kw}", flush=True)
    a, w = make_ag_inputs(cfg, i)
    a_full, c, st = mk.allgather_gemm(a.cuda(), cfg.rank, w.cuda(), opts=mk.ag_default_opts(**kw), want_stats=True)
    mk.mk_ag_gemm_status()
    assert st["status"] == 0 and st["compute_done"] == st["compute_tiles"]
    assert torch.equal(a_full.cpu(), a.reshape(cfg.m, cfg.k)), "gathered activation differs"
    a64, w64 = a.double().numpy(), w.double().numpy()
    ref_full, ref_c = oracle.allgather_gemm_reference(a64, w64, cfg.rank)
    rep = compare_gemm(c.cpu().double().numpy(), ref_c, np.abs(ref_full) @ np.abs(w64).T, cfg.k)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)
