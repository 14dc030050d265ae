"""The unfused two-stream baseline (mk_ring_attn_fwd_unfused: per-step staging and
compute launches of the same kernel on two streams, released at kernel boundaries),
through the C ABI: bitwise equal to the fused kernel run in one-step tasks, and within
the oracle's bar."""

import pytest
import torch

import oracle
import overlap_attention_amd as mk
from ring_inputs import SEQ64K, SMALL, TINY, RingConfig, make_inputs, to_f64
from tests.parity import compare, fmt, oracle_rows, wave_slice_rows

pytestmark = pytest.mark.gpu

TEST_TIMEOUT_US = 5_000_000


def announce(msg):
    print(f"[case] {msg}", flush=True)


def shape(name, n, rank, lq, lk, hq, hkv, d, causal, qk_mult=1.0):
    return RingConfig(name, rank=rank, n_chunks=n, lq=lq, lk=lk, hq=hq, hkv=hkv, d=d, causal=causal,
                      qk_mult=qk_mult)


def both(cfg, q, kv, copy_wgs):
    """(unfused out, lse), (fused one-step-task out, lse) on the same inputs."""
    copy = torch.cuda.Stream()
    o_u = torch.empty_like(q)
    l_u = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
    mk.mk_ring_attn_fwd_unfused(q, kv, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o_u, l_u, copy, copy_wgs)
    o_f, l_f = mk.ring_attn_fwd(q, kv, cfg.rank, cfg.causal, cfg.gqa_ratio,
                                opts=mk.default_opts(steps_per_task=1, tail_steps=-1, parallel_steps=-1,
                                                     spin_timeout_us=TEST_TIMEOUT_US))
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    return (o_u, l_u), (o_f, l_f)


CASES = [
    (TINY, 2),
    (SMALL, 16),
    (SMALL, 1),
    (shape("g4_causal_tail", 3, 2, 320, 320, 8, 2, 128, True, qk_mult=2.0), 4),
    (shape("g8_noncausal_12steps", 12, 5, 384, 384, 8, 1, 128, False), 3),
    (shape("ragged_d64", 5, 4, 200, 200, 6, 3, 64, True), 2),
]


@pytest.mark.parametrize("cfg,copy_wgs", CASES, ids=lambda c: c.name if hasattr(c, "name") else f"copy{c}")
def test_unfused_equals_fused_one_step_tasks_and_oracle(cfg, copy_wgs):
    announce(f"{cfg} copy_wgs={copy_wgs}")
    q, kv = make_inputs(cfg, seed=17)
    (o_u, l_u), (o_f, l_f) = both(cfg, q.cuda(), kv.cuda(), copy_wgs)
    assert torch.equal(o_u, o_f) and torch.equal(l_u, l_f)
    ref_o, ref_l = oracle.ring_attention_reference(to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio)
    rep = compare(to_f64(o_u), l_u.double().cpu().numpy(), ref_o, ref_l)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


@pytest.mark.timeout(600)
def test_unfused_full_size_64k():
    cfg = SEQ64K
    announce(f"{cfg} unfused, full size")
    q, kv = make_inputs(cfg, seed=2)
    (o_u, l_u), (o_f, l_f) = both(cfg, q.cuda(), kv.cuda(), 16)
    assert torch.equal(o_u, o_f) and torch.equal(l_u, l_f)
    rows = wave_slice_rows(cfg.lq, per_slice_random=1, seed=5)
    ref_o, ref_l = oracle_rows(oracle, to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio, rows,
                               progress=True)
    rep = compare(to_f64(o_u.cpu()[rows]), l_u.cpu()[:, rows].double().numpy(), ref_o, ref_l)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


def test_unfused_then_fused_on_one_workspace():
    a, b = SMALL, shape("other", 5, 3, 300, 300, 8, 2, 64, True)
    qa, kva = make_inputs(a, seed=21)
    qb, kvb = make_inputs(b, seed=22)
    ra = oracle.ring_attention_reference(to_f64(qa), to_f64(kva), a.rank, a.causal, a.gqa_ratio)
    rb = oracle.ring_attention_reference(to_f64(qb), to_f64(kvb), b.rank, b.causal, b.gqa_ratio)
    qa, kva, qb, kvb = qa.cuda(), kva.cuda(), qb.cuda(), kvb.cuda()
    copy = torch.cuda.Stream()
    announce("unfused, fused, unfused back to back on one stream")
    res = []
    for cfg, q, kv in ((a, qa, kva), (b, qb, kvb), (a, qa, kva)):
        o = torch.empty_like(q)
        l = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
        if len(res) == 1:
            mk.mk_ring_attn_fwd(q, kv, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o, l)
        else:
            mk.mk_ring_attn_fwd_unfused(q, kv, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o, l, copy, 8)
        res.append((o, l))
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    for (o, l), ref in zip(res, (ra, rb, ra)):
        rep = compare(to_f64(o), l.double().cpu().numpy(), *ref)
        assert rep["ok"], fmt(rep)


def test_unfused_rejects_one_stream():
    cfg = TINY
    q, kv = make_inputs(cfg, seed=1)
    q, kv = q.cuda(), kv.cuda()
    o = torch.empty_like(q)
    l = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    announce("copy stream == compute stream")
    with pytest.raises(mk.MkError) as e:
        mk.mk_ring_attn_fwd_unfused(q, kv, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o, l, s, 4, stream=s)
    assert e.value.status == mk.MK_E_INVAL
