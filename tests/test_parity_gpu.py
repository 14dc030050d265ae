"""Parity of the HIP path (called through the C ABI) with the fp64 oracle, on one GPU.

Every case prints what it runs before launching, so a failing GPU run names its case.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import overlap_attention_amd as mk
from ring_inputs import SEQ32K_D64, SEQ64K, SEQ128K, SMALL, TINY, RingConfig, make_inputs, to_f64
from tests.parity import compare, fmt, oracle_rows, wave_slice_rows

pytestmark = pytest.mark.gpu

# Every on-GPU wait is bounded well below the test timeout.
TEST_TIMEOUT_US = 5_000_000


def opts(**kw):
    kw.setdefault("spin_timeout_us", TEST_TIMEOUT_US)
    return mk.default_opts(**kw)


def announce(msg):
    print(f"[case] {msg}", flush=True)


def run_gpu(q, kv, cfg, **kw):
    want_stats = kw.pop("want_stats", False)
    res = mk.ring_attn_fwd(q, kv, cfg.rank, cfg.causal, cfg.gqa_ratio, opts=opts(**kw), want_stats=want_stats)
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    return res


def check_full(cfg, seed, **kw):
    announce(f"{cfg} seed={seed} opts={kw}")
    q, kv = make_inputs(cfg, seed)
    qg, kvg = q.cuda(), kv.cuda()
    out, lse = run_gpu(qg, kvg, cfg, **kw)
    ref_o, ref_l = oracle.ring_attention_reference(to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio)
    rep = compare(to_f64(out), lse.double().cpu().numpy(), ref_o, ref_l)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)
    return out, lse


def shape(name, n, rank, lq, lk, hq, hkv, d, causal, qk_mult=1.0):
    return RingConfig(name, rank=rank, n_chunks=n, lq=lq, lk=lk, hq=hq, hkv=hkv, d=d, causal=causal,
                      qk_mult=qk_mult)


# --------------------------------------------------------------- the five workloads

def test_tiny_workload_full():
    check_full(TINY, seed=0)


SMALL_SHAPES = [
    shape("single_key", 1, 0, 1, 1, 1, 1, 64, True),
    shape("one_row_many_steps", 5, 4, 1, 1, 2, 1, 128, True),
    shape("ragged_causal_g2", 3, 1, 200, 200, 6, 3, 64, True),
    shape("ragged_noncausal_g2", 3, 2, 200, 200, 6, 3, 64, False),
    shape("lq_ne_lk_g3", 2, 0, 77, 300, 6, 2, 128, False),
    shape("g16_ragged", 4, 3, 129, 129, 16, 1, 128, True),
    shape("d64_two_blocks", 2, 1, 513, 513, 8, 8, 64, True),
    shape("g8_noncausal", 6, 2, 384, 384, 8, 1, 128, False),
    shape("short_q_long_k", 3, 0, 64, 1000, 4, 2, 64, False),
    shape("rank0_causal", 4, 0, 256, 256, 4, 4, 128, True),
    shape("g4_causal_tail", 3, 2, 320, 320, 8, 2, 128, True, qk_mult=2.0),
]


@pytest.mark.parametrize("cfg", SMALL_SHAPES, ids=lambda c: c.name)
def test_small_shapes_full(cfg):
    check_full(cfg, seed=11)


def test_small_workload_full():
    check_full(SMALL, seed=1)


def check_full_size(cfg, seed, rows, label):
    """A full-size workload in the default launch configuration (as benchmarked),
    compared with the oracle at `rows` (None: every row), all heads."""
    announce(f"{cfg} seed={seed} {label}")
    q, kv = make_inputs(cfg, seed=seed)
    qg, kvg = q.cuda(), kv.cuda()
    out, lse, stats = run_gpu(qg, kvg, cfg, want_stats=True)
    print("    stats:", stats, flush=True)
    assert stats["status"] == 0
    assert stats["compute_tasks_done"] == stats["n_units"] * stats["n_steps"]
    assert stats["staging_tasks_done"] == stats["n_stage_tasks"]
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    out_c, lse_c = out.cpu(), lse.cpu()
    del qg, kvg, out, lse
    sel = slice(None) if rows is None else rows
    print(f"    oracle on {cfg.lq if rows is None else len(rows)} of {cfg.lq} rows, all {cfg.hq} heads", flush=True)
    ref_o, ref_l = oracle_rows(oracle, to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio, rows,
                               progress=True)
    rep = compare(to_f64(out_c[sel]), lse_c[:, sel].double().numpy(), ref_o, ref_l)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


@pytest.mark.timeout(600)
def test_full_size_64k_every_row():
    check_full_size(SEQ64K, 2, None, "every row")


@pytest.mark.timeout(600)
def test_full_size_128k_every_wave_slice():
    cfg = SEQ128K
    check_full_size(SEQ128K, 3, wave_slice_rows(cfg.lq, per_slice_random=1, seed=3), "first, last and one random row of "
                    "every 32-row slice")


@pytest.mark.timeout(600)
def test_full_size_32k_d64_every_row():
    check_full_size(SEQ32K_D64, 4, None, "every row")


SPLIT_VARIANTS = [
    dict(),
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=0),
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1),
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=2),
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1, stage_delay_ticks=3000),
    dict(grid_wgs=1),
    dict(grid_wgs=2),
    dict(grid_wgs=8),
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1, debug_flags=1),
    dict(split_mode=mk.MK_SPLIT_ADAPTIVE_PAPER),
    dict(steps_per_task=1),
    dict(steps_per_task=2),
    dict(steps_per_task=3),
    dict(steps_per_task=3, split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1, stage_delay_ticks=3000),
    dict(steps_per_task=4, grid_wgs=3),
    dict(steps_per_task=4, tail_steps=3, tail_steps_per_task=1),
    dict(steps_per_task=3, tail_steps=4, tail_steps_per_task=2, grid_wgs=5),
    dict(parallel_steps=-1),
    dict(parallel_steps=1, steps_per_task=1),
    dict(parallel_steps=1, steps_per_task=2, grid_wgs=5),
    dict(parallel_steps=1, steps_per_task=4, split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1,
         stage_delay_ticks=3000),
]


@pytest.mark.parametrize("variant", SPLIT_VARIANTS, ids=lambda v: "-".join(f"{k}{v[k]}" for k in v) or "default")
def test_many_steps_every_split_matches_oracle(variant):
    """Six ring steps, slots reused three times, one or many staging workgroups."""
    cfg = shape("g8_noncausal", 6, 2, 384, 384, 8, 1, 128, False)
    for rep in range(3):
        out, lse = check_full(cfg, seed=11, **variant)
    if variant.get("debug_flags"):
        q, kv = make_inputs(cfg, seed=11)
        st = run_gpu(q.cuda(), kv.cuda(), cfg, want_stats=True, **variant)[2]
        assert st["debug_mismatches"] == 0, st


# --------------------------------------------------------------- special cases

def test_constant_v_rows_return_v():
    cfg = shape("constv", 4, 2, 256, 256, 8, 2, 128, True)
    announce("constant V")
    q, kv = make_inputs(cfg, seed=3)
    u = torch.randn((cfg.hkv, cfg.d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    kv[:, 1] = u[None, None]
    out, _ = run_gpu(q.cuda(), kv.cuda(), cfg)
    want = u.double().repeat_interleave(cfg.gqa_ratio, dim=0)[None].expand(cfg.lq, -1, -1)
    err = (out.double().cpu() - want).abs().max().item()
    print("    max err", err, flush=True)
    assert err <= 1e-2


def test_rising_scores_take_the_rescale_path():
    """Scores that rise by about 9 nats from each KV block to the next, in ring order:
    every block after the first drives the lagging running max past its bound, and the
    packed fp16 row sum of such a block overflows to inf, so the kernel must take the
    rescale path on every block and still match the oracle."""
    cfg = shape("rising", 2, 0, 256, 256, 4, 2, 128, False)
    announce("rising scores: rescale on every block, fp16 row-sum overflow")
    q, kv = make_inputs(cfg, seed=12)
    q[:] = 0.5
    g = torch.Generator().manual_seed(13)
    order = [0, 1]  # ring order of the chunks for rank 0 of 2: local first, then chunk 1
    for pos, c in enumerate(order):
        for j in range(cfg.lk // 64):
            b = 1.6 * (pos * (cfg.lk // 64) + j)   # 0.5 * 128 * b / sqrt(128) = 5.66 b nats
            noise = 0.05 * torch.randn((64, cfg.hkv, cfg.d), generator=g)
            kv[c, 0, 64 * j:64 * (j + 1)] = (b + noise).to(torch.bfloat16)
    out, lse = run_gpu(q.cuda(), kv.cuda(), cfg)
    ref_o, ref_l = oracle.ring_attention_reference(to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio)
    rep = compare(to_f64(out), lse.double().cpu().numpy(), ref_o, ref_l)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


def test_future_chunks_never_read():
    cfg = shape("poison", 6, 2, 192, 192, 4, 2, 64, True)
    announce("causal poisoning of chunks after the rank")
    q, kv = make_inputs(cfg, seed=4)
    o1, l1 = run_gpu(q.cuda(), kv.cuda(), cfg)
    bad = kv.clone()
    bad[cfg.rank + 1:] = float("nan")
    o2, l2 = run_gpu(q.cuda(), bad.cuda(), cfg)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noncausal_rank_invariance():
    base = shape("rankinv", 4, 0, 128, 128, 4, 4, 64, False)
    q, kv = make_inputs(base, seed=6)
    announce("non-causal rank invariance")
    outs = []
    for r in range(4):
        cfg = shape("rankinv", 4, r, 128, 128, 4, 4, 64, False)
        outs.append(run_gpu(q.cuda(), kv.cuda(), cfg))
    for o, l in outs[1:]:
        assert (o.float() - outs[0][0].float()).abs().max().item() <= 1e-2
        assert ((l - outs[0][1]).abs() / outs[0][1].abs().clamp(min=1)).max().item() <= 1e-3


# --------------------------------------------------------------- protocol

def test_bitwise_identical_across_splits_grids_and_delays():
    """Within one mode the result bits do not depend on the staging split, the grid, the
    timing or the controller. The default mode of this workload runs its step groups in
    parallel (its units fill under half of the device), and that choice is the
    device's, not the grid's."""
    cfg = SMALL
    q, kv = make_inputs(cfg, seed=1)
    qg, kvg = q.cuda(), kv.cuda()
    announce("reference split")
    ref_o, ref_l = check_full(cfg, seed=1)
    st = run_gpu(qg, kvg, cfg, want_stats=True)[2]
    assert st["parallel_steps"] == 1, st
    timing = [dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=n) for n in (0, 1, 2, 4, 8, 32)]
    timing += [dict(grid_wgs=g) for g in (1, 3, 8, 37)]
    timing += [dict(stage_delay_ticks=2000), dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1,
                                                 stage_delay_ticks=5000)]
    timing += [dict(initial_staging_wgs=16, controller_period_us=1), dict(split_mode=mk.MK_SPLIT_ADAPTIVE_PAPER)]
    # Staging pieces: a tile's 16 KV heads in 1, 3 (6 + 6 + 4), 16 or 5 pieces.
    timing += [dict(stage_pieces=1), dict(stage_pieces=3), dict(stage_pieces=16, grid_wgs=37),
               dict(stage_pieces=5, split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1, stage_delay_ticks=3000)]
    for v in timing:
        announce(f"variant {v}")
        o, l = run_gpu(qg, kvg, cfg, **v)
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), v
    # Sequential mode: the blocks of a unit are processed in the same order with the
    # same arithmetic whatever the grouping (the state between tasks is stored and
    # reloaded exactly), so task sizes and tails do not change the bits either.
    announce("sequential reference")
    seq_o, seq_l = check_full(cfg, seed=1, parallel_steps=-1)
    seq = [dict(steps_per_task=g, tail_steps=-1) for g in (1, 2, 3, 4)]
    seq += [dict(steps_per_task=4, tail_steps=2, tail_steps_per_task=1), dict(grid_wgs=3), dict(grid_wgs=200)]
    seq += timing[:2]
    for v in seq:
        announce(f"sequential variant {v}")
        o, l = run_gpu(qg, kvg, cfg, parallel_steps=-1, **v)
        assert torch.equal(o, seq_o) and torch.equal(l, seq_l), v
    # Parallel mode with each grouping: the merge runs in group order, so a grouping's
    # bits do not depend on which group finishes last (grids and staging splits vary).
    for g in (1, 2, 3, 4):
        announce(f"parallel grouping {g}")
        po, pl = check_full(cfg, seed=1, parallel_steps=1, steps_per_task=g)
        for v in (dict(grid_wgs=5), dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=2, stage_delay_ticks=3000)):
            o, l = run_gpu(qg, kvg, cfg, parallel_steps=1, steps_per_task=g, **v)
            assert torch.equal(o, po) and torch.equal(l, pl), (g, v)


def test_parallel_step_groups_reuse_slots():
    """Twelve non-causal ring steps (each slot reused) with a unit's step groups run at
    once and merged: every grouping and staging split matches the oracle, and the
    parallel and sequential modes agree within the same bar."""
    cfg = shape("par_reuse", 12, 5, 320, 320, 4, 2, 64, False)
    for v in (dict(), dict(parallel_steps=1, steps_per_task=1), dict(parallel_steps=1, steps_per_task=3, grid_wgs=7),
              dict(parallel_steps=1, steps_per_task=4, split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1),
              dict(parallel_steps=1, steps_per_task=2, split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=3,
                   stage_delay_ticks=4000),
              dict(parallel_steps=-1)):
        check_full(cfg, seed=21, **v)
    q, kv = make_inputs(cfg, seed=21)
    st = run_gpu(q.cuda(), kv.cuda(), cfg, want_stats=True, parallel_steps=1, steps_per_task=2)[2]
    print("    stats:", st, flush=True)
    assert st["parallel_steps"] == 1 and st["step_groups"] == 6
    assert st["compute_tasks_done"] == st["n_units"] * st["n_steps"]


def test_parallel_step_groups_causal_gqa():
    """Causal GQA, rank 9 of 10 (ten steps, slots reused, the diagonal step in group 0):
    parallel groups of every size and a ragged head dim 128 query block, against the
    oracle; the default mode is parallel here."""
    cfg = shape("par_causal_gqa", 10, 9, 200, 200, 8, 2, 128, True)
    q, kv = make_inputs(cfg, seed=23)
    st = run_gpu(q.cuda(), kv.cuda(), cfg, want_stats=True)[2]
    assert st["parallel_steps"] == 1, st
    for v in (dict(), dict(steps_per_task=1), dict(steps_per_task=3, grid_wgs=6),
              dict(steps_per_task=4, split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=2, stage_delay_ticks=3000)):
        check_full(cfg, seed=23, parallel_steps=1, **v)


def test_staging_pieces_with_ragged_head_ranges():
    """A tile's five KV heads staged in 1, 2 (3 + 2), 3 (2 + 2 + 1) or 5 pieces, each with
    its own ready flag that only the units of its heads wait for: every split matches
    the oracle, the piece count is reported, and the bits do not depend on it."""
    cfg = shape("pieces_ragged", 6, 4, 320, 320, 10, 5, 64, True)
    q, kv = make_inputs(cfg, seed=29)
    qg, kvg = q.cuda(), kv.cuda()
    ref = None
    for pieces, want, extra in ((1, 1, {}), (2, 2, dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1,
                                                            stage_delay_ticks=3000)),
                                (3, 3, dict(grid_wgs=4)), (5, 5, {}), (9, 5, dict(parallel_steps=-1)),
                                (4, 3, dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=3, stage_delay_ticks=2000))):
        o, l = check_full(cfg, seed=29, stage_pieces=pieces, **extra)
        st = run_gpu(qg, kvg, cfg, want_stats=True, stage_pieces=pieces, **extra)[2]
        assert st["stage_pieces"] == want and st["n_stage_tasks"] == st["n_steps"] * st["n_stage_tiles"] * want, st
        assert st["staging_tasks_done"] == st["n_stage_tasks"], st
        if extra.get("parallel_steps") is None:
            if ref is None:
                ref = (o, l)
            assert torch.equal(o, ref[0]) and torch.equal(l, ref[1]), pieces


def test_back_to_back_launches_and_shape_changes():
    a = SMALL
    b = shape("other", 5, 3, 300, 300, 8, 2, 64, True)
    qa, kva = make_inputs(a, seed=21)
    qb, kvb = make_inputs(b, seed=22)
    ra = oracle.ring_attention_reference(to_f64(qa), to_f64(kva), a.rank, a.causal, a.gqa_ratio)
    rb = oracle.ring_attention_reference(to_f64(qb), to_f64(kvb), b.rank, b.causal, b.gqa_ratio)
    qa, kva, qb, kvb = qa.cuda(), kva.cuda(), qb.cuda(), kvb.cuda()
    plan = [(a, qa, kva, ra), (b, qb, kvb, rb), (a, qa, kva, ra), (a, qa, kva, ra)]
    results = []
    for i, (cfg, q, kv, _) in enumerate(plan):
        announce(f"launch {i}: {cfg.name}")
        # Enqueued back to back on one stream: the launches share one workspace.
        results.append(mk.ring_attn_fwd(q, kv, cfg.rank, cfg.causal, cfg.gqa_ratio, opts=opts()))
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    for i, ((out, lse), (_, _, _, ref)) in enumerate(zip(results, plan)):
        rep = compare(to_f64(out), lse.double().cpu().numpy(), *ref)
        assert rep["ok"], (i, fmt(rep))


def test_stale_slots_of_previous_launch_are_not_consumed():
    """Launch with inputs X, then with inputs Y and slow staging: a compute wave that
    consumed a flag of the earlier launch would read X's chunks from the slots."""
    cfg = shape("stale", 6, 5, 256, 256, 8, 4, 128, True)
    qx, kvx = make_inputs(cfg, seed=31)
    qy, kvy = make_inputs(cfg, seed=32)
    ref = oracle.ring_attention_reference(to_f64(qy), to_f64(kvy), cfg.rank, cfg.causal, cfg.gqa_ratio)
    qx, kvx, qy, kvy = qx.cuda(), kvx.cuda(), qy.cuda(), kvy.cuda()
    announce("stale slot check")
    mk.ring_attn_fwd(qx, kvx, cfg.rank, cfg.causal, cfg.gqa_ratio, opts=opts())
    out, lse = mk.ring_attn_fwd(qy, kvy, cfg.rank, cfg.causal, cfg.gqa_ratio,
                                opts=opts(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1,
                                          stage_delay_ticks=20000))
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    rep = compare(to_f64(out), lse.double().cpu().numpy(), *ref)
    assert rep["ok"], fmt(rep)


def test_wait_bound_reports_timeout_and_recovers():
    cfg = shape("timeout", 3, 2, 128, 128, 2, 2, 64, True)
    q, kv = make_inputs(cfg, seed=41)
    qg, kvg = q.cuda(), kv.cuda()
    announce("staging disabled: the bounded waits must expire")
    mk.ring_attn_fwd(qg, kvg, cfg.rank, cfg.causal, cfg.gqa_ratio,
                     opts=mk.default_opts(disable_staging=1, spin_timeout_us=100_000))
    with pytest.raises(mk.MkError) as e:
        mk.mk_ring_attn_status()
    assert e.value.status == mk.MK_E_TIMEOUT
    announce("next call on the same workspace")
    check_full(cfg, seed=41)


def group_firsts(n_steps, g, tail_steps, tail_g):
    """First step of every step group, per the rule the header documents: groups of g
    steps, the last tail_steps steps in groups of tail_g."""
    n_big = max(0, n_steps - tail_steps) // g
    firsts = [i * g for i in range(n_big)]
    t = n_big * g
    while t < n_steps:
        firsts.append(t)
        t += tail_g
    return firsts


@pytest.mark.parametrize("mode,groups", [("adaptive", (4, 0, 2)), ("paper", (4, 0, 2)), ("adaptive", (2, -1, 1)),
                                         ("adaptive", (3, 2, 1))],
                         ids=["adaptive-g4", "paper-g4", "adaptive-g2", "adaptive-g3-tail2x1"])
def test_stats_and_controller_follow_eq2(mode, groups):
    """Every controller update of a traced run sets the target Eq. (2) gives for the
    inputs it records. ADAPTIVE: R_p leaves out the last ring step's unit-steps.
    ADAPTIVE_PAPER: R_p is every unclaimed unit-step, and C_p, C_s are plain measured
    averages; the first update's R_p then equals the whole compute work minus what
    was claimed before it."""
    cfg = SMALL
    q, kv = make_inputs(cfg, seed=1)
    announce(f"traced {mode} run")
    split = mk.MK_SPLIT_ADAPTIVE if mode == "adaptive" else mk.MK_SPLIT_ADAPTIVE_PAPER
    g, tail_steps, tail_g = groups
    out, lse, st = run_gpu(q.cuda(), kv.cuda(), cfg, want_stats=True, trace=1, controller_period_us=2,
                           split_mode=split, steps_per_task=g, tail_steps=tail_steps, tail_steps_per_task=tail_g,
                           parallel_steps=-1)
    print("    stats:", st, flush=True)
    assert st["status"] == 0
    assert st["compute_tasks_done"] == st["n_units"] * st["n_steps"]
    assert st["staging_tasks_done"] == st["n_stage_tasks"]
    recs = mk.mk_ring_attn_trace()
    ctrl = [r for r in recs if r[2] == 3]
    comp = [r for r in recs if r[2] == 1]
    stage = [r for r in recs if r[2] == 2]
    assert len(comp) == st["compute_tasks_done"] and len(stage) == st["staging_tasks_done"]
    assert len(ctrl) == st["controller_updates"] and len(ctrl) >= 1
    # R_p as Eq. (2) takes it: unclaimed unit-steps, less the last ring step's in
    # ADAPTIVE mode (those follow the last staging task whatever the split).
    # This workload's units fit the grid, so the default tail is none; explicit tails
    # follow the documented rule.
    firsts = group_firsts(st["n_steps"], g, max(tail_steps, 0), tail_g)
    assert st["steps_per_task"] == g and st["step_groups"] == len(firsts), (st, firsts)
    rp_max = st["n_units"] * (st["n_steps"] - 1 if mode == "adaptive" else st["n_steps"])
    for r in ctrl:
        rp, rs, cp, cs, b, target = r[3:9]
        assert 0 <= rp <= rp_max, (r, rp_max)
        exact = oracle.controller_target(b, rp, rs, cp, cs)
        # The kernel's integer rounding (half up) and clamp to [1, min(B-1, Rs)].
        if rs <= 0:
            want = 0
        else:
            hi = min(b - 1, rs)
            want = max(min(1, hi), min(hi, math.floor(exact + 0.5)))
        # Exact ties are decided in integers by the kernel; the float may sit a hair off.
        assert target == want or abs(exact + 0.5 - round(exact + 0.5)) < 1e-9, (r, exact)
    # Every (unit, step) ran once, finishing in step order per unit.
    seen = {}
    for r in sorted(comp, key=lambda r: r[0]):
        unit, step = r[3], r[4]
        assert seen.get(unit, -1) == step - 1
        seen[unit] = step
    assert len(seen) == st["n_units"]


def test_parallel_groups_stage_interleaved():
    """Parallel step groups with no slot reused: the staging role takes every group's
    first step, then every group's second (steps 0, 2, 1, 3 for two groups of two), and
    ADAPTIVE's R_p leaves out the last step of every group."""
    cfg = SMALL
    q, kv = make_inputs(cfg, seed=1)
    announce("traced parallel run")
    out, lse, st = run_gpu(q.cuda(), kv.cuda(), cfg, want_stats=True, trace=1, controller_period_us=2)
    print("    stats:", st, flush=True)
    assert st["status"] == 0 and st["parallel_steps"] == 1 and st["step_groups"] == 2 and st["n_steps"] == 4
    per_step = st["n_stage_tasks"] // st["n_steps"]
    stage = [r for r in mk.mk_ring_attn_trace() if r[2] == 2]
    assert len(stage) == st["n_stage_tasks"]
    for r in stage:
        task, step = r[3], r[4]
        assert step == (0, 2, 1, 3)[task // per_step], r
    ctrl = [r for r in mk.mk_ring_attn_trace() if r[2] == 3]
    assert ctrl and all(0 <= r[3] <= st["n_units"] * (st["n_steps"] - st["step_groups"]) for r in ctrl)
    ref = oracle.ring_attention_reference(to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio)
    rep = compare(to_f64(out), lse.double().cpu().numpy(), *ref)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


def test_v_outside_fp16_range_reports_unsupported():
    """The PV product takes V in fp16: a V the fp16 format cannot hold (|v| >= 65536 or
    not finite) in a chunk the call reads ends the launch through the error path and is
    reported as MK_E_UNSUPPORTED; the next call on the same workspace runs normally."""
    cfg = shape("vrange", 4, 3, 256, 256, 4, 2, 128, True)
    q, kv = make_inputs(cfg, seed=8)
    for where, val in (((1, 1, 77, 1, 5), 1e5), ((3, 1, 200, 0, 100), float("nan")),
                       ((0, 1, 3, 1, 0), float("-inf"))):
        bad = kv.clone()
        bad[where] = val
        announce(f"V[{where}] = {val}")
        out, lse, st = mk.ring_attn_fwd(q.cuda(), bad.cuda(), cfg.rank, cfg.causal, cfg.gqa_ratio,
                                        opts=opts(), want_stats=True)
        assert st["status"] == mk.MK_E_UNSUPPORTED, st
        with pytest.raises(mk.MkError) as e:
            mk.mk_ring_attn_status()
        assert e.value.status == mk.MK_E_UNSUPPORTED
        announce("next call on the same workspace")
        check_full(cfg, seed=8)


def test_host_written_stale_and_future_flags_are_not_consumed():
    """Every ready flag and unit flag holds, before the launch, a stamp of the right
    step but of the previous or the next launch; the slots hold an earlier launch's
    data; staging is slow. A consumed flag would read that data."""
    cfg = shape("flagtable", 6, 5, 256, 256, 8, 4, 128, True)
    qx, kvx = make_inputs(cfg, seed=33)
    qy, kvy = make_inputs(cfg, seed=34)
    ref = oracle.ring_attention_reference(to_f64(qy), to_f64(kvy), cfg.rank, cfg.causal, cfg.gqa_ratio)
    qx, kvx, qy, kvy = qx.cuda(), kvx.cuda(), qy.cuda(), kvy.cuda()
    announce("host-written stale and future flags")
    mk.ring_attn_fwd(qx, kvx, cfg.rank, cfg.causal, cfg.gqa_ratio, opts=opts())
    out, lse = mk.ring_attn_fwd(qy, kvy, cfg.rank, cfg.causal, cfg.gqa_ratio,
                                opts=opts(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1,
                                          stage_delay_ticks=20000, debug_flags=2))
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    rep = compare(to_f64(out), lse.double().cpu().numpy(), *ref)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


def test_host_pointer_rejected():
    cfg = shape("hostptr", 2, 1, 128, 128, 2, 2, 64, True)
    q, kv = make_inputs(cfg, seed=51)
    out = torch.empty_like(q).cuda()
    lse = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
    announce("host pointer")
    with pytest.raises(mk.MkError) as e:
        mk.mk_ring_attn_fwd(q, kv.cuda(), cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, out, lse)
    assert e.value.status == mk.MK_E_INVAL
