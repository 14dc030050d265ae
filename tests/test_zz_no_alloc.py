"""The entry point that allocates nothing (mk_ring_attn_fwd_noalloc), called through
the C ABI, against the existing entry point (mk_ring_attn_fwd) on the same inputs:
two calls in a row, the second smaller, each compared element by element with the
existing entry point's result and with the oracle. Also: a problem whose state does
not fit the fixed scratch array is refused on the host."""

import pytest
import torch

import oracle
import overlap_attention_amd as mk
from ring_inputs import RingConfig, make_inputs, to_f64
from tests.parity import compare, fmt

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)


def run_both(cfg, seed):
    q, kv = make_inputs(cfg, seed)
    qg, kvg = q.cuda(), kv.cuda()
    o_ref = torch.empty_like(qg)
    l_ref = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
    o_na = torch.empty_like(qg)
    l_na = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
    announce(f"{cfg.name}: mk_ring_attn_fwd")
    mk.mk_ring_attn_fwd(qg, kvg, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o_ref, l_ref)
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    announce(f"{cfg.name}: mk_ring_attn_fwd_noalloc")
    mk.mk_ring_attn_fwd_noalloc(qg, kvg, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o_na, l_na)
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    # Same kernel, same decomposition: the results are identical, not merely close.
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
    ref_o, ref_l = oracle.ring_attention_reference(to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio)
    rep = compare(to_f64(o_na), l_na.double().cpu().numpy(), ref_o, ref_l)
    print("   ", fmt(rep), flush=True)
    assert rep["ok"], fmt(rep)


def test_noalloc_matches_the_allocating_entry_point_twice_second_smaller():
    big = RingConfig("noalloc_big_r3of4_L512_h8kv2_d128_causal", rank=3, n_chunks=4, lq=512, lk=512, hq=8, hkv=2,
                     d=128, causal=True)
    small = RingConfig("noalloc_small_r1of3_L200_h4kv4_d64_nc", rank=1, n_chunks=3, lq=200, lk=200, hq=4, hkv=4,
                       d=64, causal=False)
    run_both(big, seed=61)
    run_both(small, seed=62)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    cfg = RingConfig("noalloc_too_big", rank=15, n_chunks=16, lq=8192, lk=8192, hq=32, hkv=8, d=128, causal=True)
    q = torch.zeros((cfg.lq, cfg.hq, cfg.d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((cfg.n_chunks, 2, cfg.lk, cfg.hkv, cfg.d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
    announce("too big for the scratch array")
    with pytest.raises(mk.MkError) as e:
        mk.mk_ring_attn_fwd_noalloc(q, kv, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, out, lse)
    assert e.value.status == mk.MK_E_UNSUPPORTED
    assert "bytes of device state" in str(e.value)
