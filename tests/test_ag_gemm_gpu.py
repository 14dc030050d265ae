"""Parity of one rank's AllGather+GEMM (HIP path, through the C ABI) with the fp64
oracle, on one GPU: the gathered activation bit for bit, the product within the GEMM
bar of tests/parity.py (half a bf16 ulp plus the fp32 accumulation bound).

Every case prints what it runs before launching, so a failing GPU run names its case.
"""

import numpy as np
import pytest
import torch

import oracle
import overlap_attention_amd as mk
from ag_inputs import AG_HEADLINE, AG_TINY, AgConfig, make_ag_inputs
from tests.parity import compare_gemm, fmt

pytestmark = pytest.mark.gpu

TEST_TIMEOUT_US = 5_000_000


def announce(msg):
    print(f"[case] {msg}", flush=True)


def opts(**kw):
    kw.setdefault("spin_timeout_us", TEST_TIMEOUT_US)
    return mk.ag_default_opts(**kw)


def run_gpu(cfg, a, w, **kw):
    want_stats = kw.pop("want_stats", False)
    res = mk.allgather_gemm(a, cfg.rank, w, opts=opts(**kw), want_stats=want_stats)
    torch.cuda.synchronize()
    mk.mk_ag_gemm_status()
    return res


def check(cfg, seed, rows=None, **kw):
    """Runs the config and checks A_full bitwise and C against the oracle (at `rows`
    of the gathered matrix, or every row)."""
    announce(f"{cfg} seed={seed} opts={kw}")
    a, w = make_ag_inputs(cfg, seed)
    a_full, c = run_gpu(cfg, a.cuda(), w.cuda(), **kw)
    assert torch.equal(a_full.cpu(), a.reshape(cfg.m, cfg.k)), "gathered activation differs"
    a64 = a.double().numpy()
    w64 = w.double().numpy()
    sel = np.arange(cfg.m) if rows is None else np.asarray(rows)
    ref_full, ref_c = oracle.allgather_gemm_reference(a64, w64, cfg.rank)
    abs_sum = np.abs(ref_full[sel]) @ np.abs(w64).T
    rep = compare_gemm(c.cpu().double().numpy()[sel], ref_c[sel], abs_sum, cfg.k)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)
    return a_full, c


SHAPES = [
    AG_TINY,
    AgConfig("ragged_r2of3_M200_K192_N520", n_ranks=3, rank=2, m_loc=200, k=192, n_out=520),
    AgConfig("one_row_r0of5_K64_N8", n_ranks=5, rank=0, m_loc=1, k=64, n_out=8),
    AgConfig("single_rank_M300_K64_N1024", n_ranks=1, rank=0, m_loc=300, k=64, n_out=1024),
    AgConfig("two_chunks_r1of2_M130_K128_N1536", n_ranks=2, rank=1, m_loc=130, k=128, n_out=1536),
    AgConfig("many_ranks_r9of16_M64_K256_N512", n_ranks=16, rank=9, m_loc=64, k=256, n_out=512),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_shapes_match_oracle(cfg):
    check(cfg, seed=3)


SPLITS = [
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=0),
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1),
    dict(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=4),
    dict(split_mode=mk.MK_SPLIT_ADAPTIVE_PAPER),
    dict(grid_wgs=1),
    dict(grid_wgs=3),
    dict(grid_wgs=8),
    dict(initial_staging_wgs=16, controller_period_us=1),
]


def test_splits_and_grids_bitwise_identical():
    cfg = AgConfig("splits_r2of4_M384_K512_N1024", n_ranks=4, rank=2, m_loc=384, k=512, n_out=1024)
    ref_full, ref_c = check(cfg, seed=5)
    a, w = make_ag_inputs(cfg, 5)
    a, w = a.cuda(), w.cuda()
    for v in SPLITS:
        announce(f"variant {v}")
        f, c = run_gpu(cfg, a, w, **v)
        assert torch.equal(f, ref_full) and torch.equal(c, ref_c), v


def test_stale_flags_of_previous_launch_are_not_consumed():
    """Launch on inputs X, then on inputs Y with one slow staging workgroup: a tile that
    consumed a flag of the earlier launch would read X's rows from a_full."""
    cfg = AgConfig("stale_r3of4_M256_K256_N512", n_ranks=4, rank=3, m_loc=256, k=256, n_out=512)
    ax, wx = make_ag_inputs(cfg, 7)
    ay, wy = make_ag_inputs(cfg, 8)
    announce("stale flags")
    fx, cx = mk.allgather_gemm(ax.cuda(), cfg.rank, wx.cuda(), opts=opts())
    # Y writes into X's a_full and c: the same addresses, so stale rows would show.
    mk.mk_allgather_gemm_ex(ay.cuda(), cfg.n_ranks, cfg.rank, wy.cuda(), fx, cx,
                            opts=opts(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=1, grid_wgs=4))
    torch.cuda.synchronize()
    mk.mk_ag_gemm_status()
    assert torch.equal(fx.cpu(), ay.reshape(cfg.m, cfg.k))
    ref_full, ref_c = oracle.allgather_gemm_reference(ay.double().numpy(), wy.double().numpy(), cfg.rank)
    rep = compare_gemm(cx.cpu().double().numpy(), ref_c, np.abs(ref_full) @ np.abs(wy.double().numpy()).T, cfg.k)
    assert rep["ok"], fmt(rep)


def test_unfused_phases_equal_the_fused_call():
    """The unfused sequence of the same code (gather, then GEMM, two launches on one
    stream) writes the fused call's bits; a GEMM phase without its gather, or after a
    gather with other arguments, is refused on the host."""
    cfg = AgConfig("phases_r1of4_M320_K256_N768", n_ranks=4, rank=1, m_loc=320, k=256, n_out=768)
    a, w = make_ag_inputs(cfg, 11)
    a, w = a.cuda(), w.cuda()
    announce("fused reference")
    ref_full, ref_c = check(cfg, seed=11)
    f = torch.empty((cfg.m, cfg.k), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((cfg.m, cfg.n_out), dtype=torch.bfloat16, device="cuda")
    for g in (0, 5):
        announce(f"phases, grid {g}")
        f.zero_()
        c.zero_()
        mk.mk_allgather_gemm_ex(a, cfg.n_ranks, cfg.rank, w, f, c, opts=opts(phase=1, grid_wgs=g))
        torch.cuda.synchronize()
        assert torch.equal(f, ref_full) and not c.any(), "the gather phase writes A_full only"
        mk.mk_allgather_gemm_ex(a, cfg.n_ranks, cfg.rank, w, f, c, opts=opts(phase=2, grid_wgs=g))
        torch.cuda.synchronize()
        mk.mk_ag_gemm_status()
        assert torch.equal(f, ref_full) and torch.equal(c, ref_c), g
    announce("GEMM phase without its gather")
    with pytest.raises(RuntimeError):
        mk.mk_allgather_gemm_ex(a, cfg.n_ranks, cfg.rank, w, f, c, opts=opts(phase=2))
    mk.mk_allgather_gemm_ex(a, cfg.n_ranks, cfg.rank, w, f, c, opts=opts(phase=1))
    other = torch.zeros_like(c)
    with pytest.raises(RuntimeError):
        mk.mk_allgather_gemm_ex(a, cfg.n_ranks, cfg.rank, w, f, other, opts=opts(phase=2))
    torch.cuda.synchronize()
    mk.mk_ag_gemm_status()


def test_stats_count_every_task():
    cfg = AgConfig("stats_r1of8_M256_K256_N1024", n_ranks=8, rank=1, m_loc=256, k=256, n_out=1024)
    a, w = make_ag_inputs(cfg, 9)
    announce("stats")
    _, _, st = run_gpu(cfg, a.cuda(), w.cuda(), want_stats=True)
    print("    stats:", st, flush=True)
    assert st["status"] == 0
    assert st["compute_done"] == st["compute_tiles"] == 8 * 1 * 4  # ranks x 256-row tiles x 256-column tiles
    assert st["staging_done"] == st["staging_tasks"] == 8 * 2 * 2  # ranks x chunks x 64-row pieces


@pytest.mark.timeout(600)
def test_wait_bound_reports_timeout_and_recovers():
    cfg = AgConfig("timeout_r1of3_M200_K128_N256", n_ranks=3, rank=1, m_loc=200, k=128, n_out=256)
    a, w = make_ag_inputs(cfg, 11)
    announce("staging disabled: the waits for remote shards must expire")
    mk.allgather_gemm(a.cuda(), cfg.rank, w.cuda(), opts=mk.ag_default_opts(disable_staging=1, spin_timeout_us=100_000))
    with pytest.raises(mk.MkError) as e:
        mk.mk_ag_gemm_status()
    assert e.value.status == mk.MK_E_TIMEOUT
    announce("next call on the same workspace")
    check(cfg, seed=11)


def test_full_size_headline_sampled_rows():
    """The 16K-row, K=8192, N=4096 rank share in the default launch configuration: the
    whole gathered activation bit for bit, and C at the first, last and one random row
    of every 128-row chunk, every column."""
    cfg = AG_HEADLINE
    announce(f"{cfg} full size")
    a, w = make_ag_inputs(cfg, 1)
    a_full, c, st = run_gpu(cfg, a.cuda(), w.cuda(), want_stats=True)
    print("    stats:", st, flush=True)
    assert st["status"] == 0 and st["compute_done"] == st["compute_tiles"]
    assert torch.equal(a_full.cpu(), a.reshape(cfg.m, cfg.k))
    rng = np.random.default_rng(11)
    rows = sorted({r for c0 in range(0, cfg.m, 128) for r in (c0, min(cfg.m, c0 + 128) - 1,
                                                              int(rng.integers(c0, min(cfg.m, c0 + 128))))})
    print(f"    oracle on {len(rows)} of {cfg.m} rows", flush=True)
    a64 = a.reshape(cfg.m, cfg.k)[rows].double().numpy()
    w64 = w.double().numpy()
    # The oracle on the sampled rows, posed as one shard holding just those rows.
    _, ref = oracle.allgather_gemm_reference(a64[None], w64, 0)
    rep = compare_gemm(c.cpu()[rows].double().numpy(), ref, np.abs(a64) @ np.abs(w64).T, cfg.k)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)
