"""Benchmark of the per-rank ring-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R] [--workload NAME]
                    [--no-cpu-baseline] [--sweep] [--size-sweep] [--unfused] [--verify]
                    [--copy-calibration-mib M]
    python bench.py --traffic-from DIR [--copy-calibration-mib M]   (no GPU)
    python bench.py --probes    (MFMA-stream, vector-ALU, LDS-read and co-execution probes; prints a table)

A step is one call of mk_ring_attn_fwd: the whole hot path (every ring step of one
rank, staging included) over one batch of synthetic input already resident in HBM.
W untimed warm-up calls, then K calls enqueued back to back on one stream with one
synchronisation at the end (the measurement protocol of the mKernel paper, §5.1),
timed with HIP events recorded on that stream; the K calls are also timed in R groups
(median and min per launch). Prints ONE JSON line on stdout.

The default workload is the per-rank share of a 64K-token causal GQA sequence over
16 ranks (rank 15: the slowest rank of a contiguous causal ring). Throughput counts
algorithmic FLOPs only: 4 * D * Hq * (visible query-key pairs).
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and % bf16 MFMA peak, per-rank ring-attn fwd, 1 MI355X"
# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
PEAK_CLOCK_GHZ = 2.4      # the clock the dense bf16 peak is quoted at
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["overlap_attention_amd/csrc/mkra_kernel.hip", "overlap_attention_amd/csrc/mkra_args.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_flops(cfg):
    if cfg.causal:
        pairs = cfg.rank * cfg.lq * cfg.lk + cfg.lq * (cfg.lq + 1) // 2
    else:
        pairs = cfg.n_chunks * cfg.lq * cfg.lk
    return 4 * cfg.d * cfg.hq * pairs


def algorithmic_bytes(cfg):
    """Q + the KV chunks read once + staged copies (read + write of the non-local
    chunks the ring moves) + out + lse."""
    q = cfg.lq * cfg.hq * cfg.d * 2
    chunk = 2 * cfg.lk * cfg.hkv * cfg.d * 2
    steps = cfg.n_steps
    return q + steps * chunk + 2 * (steps - 1) * chunk + q + cfg.hq * cfg.lq * 4


def stored_traffic(workload):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/), if they were
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_sha") != kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_rows(run_dir):
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {run_dir}")
    return rows


def _per_dispatch(rows, counter, kernel_sub):
    """Values of `counter` for the dispatches whose kernel name contains kernel_sub,
    in dispatch order."""
    sel = [r for r in rows if r["Counter_Name"] == counter and kernel_sub in r["Kernel_Name"]]
    sel.sort(key=lambda r: int(r.get("Dispatch_Id", 0) or 0))
    return [float(r["Counter_Value"]) for r in sel]


def _copy_dispatch(rows, counter):
    """Mean value of `counter` over the largest plain device copies (rocclr copyBuffer
    dispatches of the largest grid): the known-size reference."""
    copies = [r for r in rows if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    if not copies:
        return None
    gmax = max(int(r["Grid_Size"]) for r in copies)
    cal = [float(r["Counter_Value"]) for r in copies if int(r["Grid_Size"]) == gmax]
    return sum(cal) / len(cal)


def write_traffic(cfg, pmc_dir, copy_mib):
    """HBM bytes per launch of the ring kernel from rocprofv3 --pmc runs of
    `bench.py --copy-calibration-mib M`, one counter set per sub-directory of pmc_dir:
      dram/  TCC_EA0_RDREQ_DRAM_32B_sum, TCC_EA0_WRREQ_WRITE_DRAM_32B_sum: L2-to-memory
             reads and writes in 32-byte units (a 64-byte request counts 2, a 128-byte
             one 4), so bytes = 32 x count with no calibration;
      fetch/ FETCH_SIZE and write/ WRITE_SIZE (KiB by rocprofv3's derived formulas),
             each scaled by what it reads for the plain copy of M MiB in the same run;
      req/   TCC_BUBBLE_sum, TCC_EA0_RDREQ_128B_sum, TCC_EA0_RDREQ_sum,
             TCC_EA0_RDREQ_32B_sum: the request-size mix FETCH_SIZE's formula is built
             from (reported for the copy and the ring kernel).
    The ring kernel's value per launch is the median over its dispatches after the
    first. The 32-byte counters give hbm_bytes_per_launch when present."""
    import statistics as st

    res = {"copy_calibration_mib": copy_mib}
    moved = copy_mib * 1024.0 * 1024.0

    def med(v):
        return st.median(v[1:] if len(v) > 1 else v)

    sub = os.path.join(pmc_dir, "dram")
    if os.path.isdir(sub):
        rows = _counter_rows(sub)
        d = {}
        for counter, key in (("TCC_EA0_RDREQ_DRAM_32B_sum", "read"), ("TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", "write")):
            ring = _per_dispatch(rows, counter, "ring_attn_kernel")
            cp = _copy_dispatch(rows, counter)
            d[key] = {"counter": counter, "ring_bytes_per_launch": 32.0 * med(ring), "dispatches": len(ring),
                      "copy_bytes": 32.0 * cp if cp is not None else None,
                      "copy_over_moved": round(32.0 * cp / moved, 4) if cp is not None else None}
        res["dram_32b"] = d
    for name, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        sub = os.path.join(pmc_dir, name)
        if not os.path.isdir(sub):
            continue
        rows = _counter_rows(sub)
        ring = _per_dispatch(rows, counter, "ring_attn_kernel")
        cp = _copy_dispatch(rows, counter)
        scale = (copy_mib * 1024.0) / cp
        res[counter] = {"ring_kib_per_dispatch": med(ring), "dispatches": len(ring), "copy_kib_per_dispatch": cp,
                        "scale": scale, "bytes_per_launch": med(ring) * 1024.0 * scale}
    sub = os.path.join(pmc_dir, "req")
    if os.path.isdir(sub):
        rows = _counter_rows(sub)
        mix = {}
        for counter in ("TCC_BUBBLE_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum"):
            ring = _per_dispatch(rows, counter, "ring_attn_kernel")
            mix[counter] = {"ring_per_launch": med(ring) if ring else None, "copy": _copy_dispatch(rows, counter)}
        res["read_request_mix"] = mix
    if "dram_32b" in res:
        total = res["dram_32b"]["read"]["ring_bytes_per_launch"] + res["dram_32b"]["write"]["ring_bytes_per_launch"]
        res["source"] = "TCC_EA0_RDREQ_DRAM_32B_sum + TCC_EA0_WRREQ_WRITE_DRAM_32B_sum, x 32 bytes"
    else:
        total = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
        res["source"] = "FETCH_SIZE + WRITE_SIZE, copy-calibrated"
    out = {"workload": cfg.name, "kernel": "mkra::ring_attn_kernel<%d>" % cfg.d, "kernel_sha": kernel_hash(),
           "counters": res, "hbm_bytes_per_launch": int(total), "algorithmic_bytes": algorithmic_bytes(cfg)}
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    log(f"[bench] wrote {path}: {total / 1e6:.1f} MB per launch ({res['source']})")


def staging_summary(cfg, stats, ms):
    """The staging role's traffic: every step's chunk read once from its home and
    written once into the slot ring, in tiles of 128 rows."""
    chunk = 2 * cfg.lk * cfg.hkv * cfg.d * 2
    moved = 2 * cfg.n_steps * chunk  # read + write
    busy_s = stats["staging_busy_ticks"] * 1e-8
    return {
        "initial_target": stats["initial_target"],
        "final_target": stats["final_target"],
        "max_staging_wgs": stats["max_staging_wgs"],
        "grid_wgs": stats["grid_wgs"],
        "tasks": stats["staging_tasks_done"],
        "assisted_tasks": stats["assist_tasks"],
        "bytes_per_launch": moved,
        "gbs_over_launch": round(moved / (ms * 1e-3) / 1e9, 1),
        "gbs_per_busy_wg": round(moved / busy_s / 1e9, 1) if busy_s > 0 else None,
    }


SPLITS = (1, 2, 4, 8, 16, 32, 64)


def split_sweep(mk, timed, k):
    """Fixed numbers of staging workgroups against the adaptive controller: ms per
    launch and each one's latency relative to the best fixed split (Fig. 3 of the
    paper plots this ratio)."""
    res = {}
    for n in SPLITS:
        res[f"fixed{n}"] = timed(k, mk.default_opts(split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=n))[0]
    res["adaptive"] = timed(k)[0]
    res["adaptive_paper"] = timed(k, mk.default_opts(split_mode=mk.MK_SPLIT_ADAPTIVE_PAPER))[0]
    best_name = min((n for n in res if not n.startswith("adaptive")), key=lambda n: res[n])
    return {"ms": {n: round(v, 4) for n, v in res.items()}, "best_fixed": best_name,
            "best_fixed_ms": round(res[best_name], 4), "adaptive_over_best": round(res["adaptive"] / res[best_name], 3),
            "adaptive_paper_over_best": round(res["adaptive_paper"] / res[best_name], 3)}


def run_size_sweep(torch, mk, make_inputs, stream):
    """The split sweep over total sequence sizes 6K..192K (the range of Fig. 3): rank
    15 of a 16-rank causal GQA ring, Hq = 32, Hkv = 8, D = 128."""
    from ring_inputs import RingConfig

    out = []
    for total in SWEEP_SIZES:
        L = total // 16
        cfg = RingConfig(f"seq{total // 1024}k_r15of16_L{L}_h32kv8_d128_causal", rank=15, n_chunks=16, lq=L, lk=L,
                         hq=32, hkv=8, d=128, causal=True)
        q, kv = make_inputs(cfg, seed=7)
        qg, kvg = q.cuda(), kv.cuda()
        del q, kv
        o = torch.empty_like(qg)
        l = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")

        def timed_cfg(k, opts=None, groups=1):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(2):
                mk.mk_ring_attn_fwd_ex(qg, kvg, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o, l,
                                       stream=stream, opts=opts)
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(k):
                mk.mk_ring_attn_fwd_ex(qg, kvg, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o, l,
                                       stream=stream, opts=opts)
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / k, None

        k = max(3, int(60 / max(1.0, (L / 4096) ** 2 * 4.2)))
        sw = split_sweep(mk, timed_cfg, k)
        mk.mk_ring_attn_status()
        sw["tflops_adaptive"] = round(algorithmic_flops(cfg) / (sw["ms"]["adaptive"] * 1e-3) / 1e12, 1)
        sw["total_seq"] = total
        sw["chunk_rows"] = L
        out.append(sw)
        log(f"[bench] size {total}: adaptive {sw['ms']['adaptive']:.3f} ms ({sw['tflops_adaptive']} TFLOP/s), "
            f"best fixed {sw['best_fixed']} {sw['best_fixed_ms']:.3f} ms, adaptive/best {sw['adaptive_over_best']}, "
            f"paper Eq. (2)/best {sw['adaptive_paper_over_best']}")
        del qg, kvg, o, l
        torch.cuda.empty_cache()
    return out


SWEEP_SIZES = (6144, 12288, 24576, 49152, 98304, 196608)
COPY_WGS = (4, 8, 16, 32)


def run_unfused_sweep(torch, mk, make_inputs, stream, sizes=SWEEP_SIZES):
    """The fused kernel against the unfused two-stream baseline (per-step staging and
    compute launches, chunks released at kernel boundaries: Figure 1(b) of the paper)
    over total sequence sizes 6K..192K: rank 15 of a 16-rank causal GQA ring, Hq = 32,
    Hkv = 8, D = 128. The unfused leg takes the best of COPY_WGS staging workgroups.
    Returns rows and logs a markdown table."""
    from ring_inputs import RingConfig

    copy = torch.cuda.Stream()
    rows = []
    for total in sizes:
        L = total // 16
        cfg = RingConfig(f"seq{total // 1024}k_r15of16_L{L}_h32kv8_d128_causal", rank=15, n_chunks=16, lq=L, lk=L,
                         hq=32, hkv=8, d=128, causal=True)
        q, kv = make_inputs(cfg, seed=7)
        qg, kvg = q.cuda(), kv.cuda()
        del q, kv
        o = torch.empty_like(qg)
        lse = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")

        def timed_call(fn, k):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(k):
                fn()
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / k

        k = max(3, min(50, int(60 / max(1.0, (L / 4096) ** 2 * 4.2))))
        args = (qg, kvg, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, o, lse)
        fused = timed_call(lambda: mk.mk_ring_attn_fwd(*args, stream=stream), k)
        paper = timed_call(lambda: mk.mk_ring_attn_fwd_ex(
            *args, stream=stream, opts=mk.default_opts(split_mode=mk.MK_SPLIT_ADAPTIVE_PAPER)), k)
        unf = {n: timed_call(lambda: mk.mk_ring_attn_fwd_unfused(*args, copy, n, stream=stream), k) for n in COPY_WGS}
        mk.mk_ring_attn_status(stream)
        best = min(unf, key=unf.get)
        flops = algorithmic_flops(cfg)
        rows.append({"total_seq": total, "chunk_rows": L, "fused_ms": round(fused, 4),
                     "fused_paper_eq2_ms": round(paper, 4),
                     "unfused_ms": {str(n): round(v, 4) for n, v in unf.items()}, "unfused_best_copy_wgs": best,
                     "unfused_best_ms": round(unf[best], 4), "unfused_over_fused": round(unf[best] / fused, 3),
                     "fused_tflops": round(flops / (fused * 1e-3) / 1e12, 1),
                     "unfused_tflops": round(flops / (unf[best] * 1e-3) / 1e12, 1)})
        log(f"[bench] unfused size {total}: fused {fused:.3f} ms, paper Eq. (2) {paper:.3f} ms, unfused best "
            f"{unf[best]:.3f} ms ({best} copy WGs), unfused/fused {unf[best] / fused:.3f}")
        del qg, kvg, o, lse
        torch.cuda.empty_cache()
    table = ["| total tokens | chunk rows | fused ms | fused, paper Eq. (2) ms | unfused best ms (copy WGs) | "
             "unfused / fused | fused TFLOP/s | unfused TFLOP/s |", "|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        table.append(f"| {r['total_seq']} | {r['chunk_rows']} | {r['fused_ms']:.3f} | {r['fused_paper_eq2_ms']:.3f} | "
                     f"{r['unfused_best_ms']:.3f} ({r['unfused_best_copy_wgs']}) | {r['unfused_over_fused']:.3f} | "
                     f"{r['fused_tflops']} | {r['unfused_tflops']} |")
    log("\n".join(table))
    return rows


AG_METRIC = "AllGather+GEMM TFLOP/s and % bf16 MFMA peak, one rank of a tensor-parallel group, 1 MI355X"
AG_SIZES = (4096, 8192, 16384, 32768)


def run_ag(args):
    """One rank's AllGather+GEMM (C = A_full W^T after gathering the shards): the fused
    persistent kernel against the unfused baseline (the gather as one device copy, then
    the library GEMM, torch.matmul on hipBLASLt, on the same stream), over the gathered
    sizes of the mKernel paper's AllGather+GEMM results (Figure 4: 4K-32K rows; here 8
    ranks, K 8192, N 4096), with a staging split sweep on the named workload. Prints
    one JSON line."""
    import torch

    import overlap_attention_amd as mk
    from ag_inputs import AG_CONFIG_BY_NAME, AG_HEADLINE, ag_sweep_config, make_ag_inputs

    cfg = AG_CONFIG_BY_NAME[args.ag_workload] if args.ag_workload else AG_HEADLINE
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def setup(c):
        a, w = make_ag_inputs(c, seed=1)
        a, w = a.cuda(), w.cuda()
        a_full = torch.empty((c.m, c.k), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((c.m, c.n_out), dtype=torch.bfloat16, device="cuda")
        return a, w, a_full, out

    def timed(fn, k):
        # Warm-up: at least `--warmup` launches and about 0.3 s of work, so the first timed
        # region does not run at the idle clock.
        t_end = time.perf_counter() + 0.3
        n = 0
        while n < max(args.warmup, 3) or time.perf_counter() < t_end:
            fn()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(k):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / k

    def fused_fn(c, a, w, a_full, out, o=None):
        return lambda: mk.mk_allgather_gemm_ex(a, c.n_ranks, c.rank, w, a_full, out, stream=stream, opts=o)

    def unfused_fn(c, a, w, a_full, out):
        def f():
            a_full.copy_(a.reshape(c.m, c.k))
            torch.matmul(a_full, w.t(), out=out)
        return f

    gather_o = mk.ag_default_opts(phase=1)
    gemm_o = mk.ag_default_opts(phase=2)

    def same_code_fn(c, a, w, a_full, out):
        # The unfused sequence of the fused kernel's own code: the gather, then the GEMM.
        def f():
            mk.mk_allgather_gemm_ex(a, c.n_ranks, c.rank, w, a_full, out, stream=stream, opts=gather_o)
            mk.mk_allgather_gemm_ex(a, c.n_ranks, c.rank, w, a_full, out, stream=stream, opts=gemm_o)
        return f

    def gemm_only_ms(c, a, w, a_full, out, k):
        # The GEMM phase alone: events around it, the gather before each outside them.
        same_code_fn(c, a, w, a_full, out)()
        torch.cuda.synchronize()
        tot = 0.0
        for _ in range(k):
            mk.mk_allgather_gemm_ex(a, c.n_ranks, c.rank, w, a_full, out, stream=stream, opts=gather_o)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            mk.mk_allgather_gemm_ex(a, c.n_ranks, c.rank, w, a_full, out, stream=stream, opts=gemm_o)
            e1.record(stream)
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / k

    a, w, a_full, out = setup(cfg)
    flops = 2 * cfg.m * cfg.n_out * cfg.k
    ms = timed(fused_fn(cfg, a, w, a_full, out), args.steps)
    mk.mk_ag_gemm_status(stream)
    st = mk.mk_allgather_gemm_ex(a, cfg.n_ranks, cfg.rank, w, a_full, out, stream=stream, want_stats=True)
    ms_unf = timed(unfused_fn(cfg, a, w, a_full, out), args.steps)
    ms_same = timed(same_code_fn(cfg, a, w, a_full, out), args.steps)
    ms_gemm = gemm_only_ms(cfg, a, w, a_full, out, args.steps)
    mk.mk_ag_gemm_status(stream)
    log(f"[bench] ag unfused, same code: {ms_same:.4f} ms (GEMM phase alone {ms_gemm:.4f} ms)")
    tflops = flops / (ms * 1e-3) / 1e12
    clock = st["wg_cycles"] / st["wg_ticks"] * 0.1 if st["wg_ticks"] else None
    log(f"[bench] ag {cfg.name}: fused {ms:.4f} ms ({tflops:.1f} TFLOP/s), unfused {ms_unf:.4f} ms, stats {st}")
    split = {}
    for n in (1, 2, 4, 8, 16, 32):
        split[f"fixed{n}"] = round(timed(fused_fn(cfg, a, w, a_full, out, mk.ag_default_opts(
            split_mode=mk.MK_SPLIT_FIXED, fixed_staging_wgs=n)), max(3, args.steps // 3)), 4)
    split["adaptive"] = round(ms, 4)
    split["adaptive_paper"] = round(timed(fused_fn(cfg, a, w, a_full, out, mk.ag_default_opts(
        split_mode=mk.MK_SPLIT_ADAPTIVE_PAPER)), max(3, args.steps // 3)), 4)
    best = min((k for k in split if k.startswith("fixed")), key=split.get)
    log("[bench] ag split sweep: " + ", ".join(f"{k}={v:.3f}" for k, v in split.items()))
    del a, w, a_full, out
    torch.cuda.empty_cache()
    sweep = []
    if args.ag_sweep:
        for m in AG_SIZES:
            c = ag_sweep_config(m)
            a, w, a_full, out = setup(c)
            f = 2 * c.m * c.n_out * c.k
            k = max(5, min(50, int(20 / (m / 16384))))
            t_f = timed(fused_fn(c, a, w, a_full, out), k)
            t_u = timed(unfused_fn(c, a, w, a_full, out), k)
            t_s = timed(same_code_fn(c, a, w, a_full, out), k)
            mk.mk_ag_gemm_status(stream)
            sweep.append({"m": m, "fused_ms": round(t_f, 4), "unfused_ms": round(t_u, 4),
                          "unfused_over_fused": round(t_u / t_f, 3), "fused_tflops": round(f / t_f / 1e9, 1),
                          "unfused_tflops": round(f / t_u / 1e9, 1), "unfused_same_code_ms": round(t_s, 4),
                          "same_code_over_fused": round(t_s / t_f, 3)})
            log(f"[bench] ag M={m}: fused {t_f:.4f} ms ({f / t_f / 1e9:.1f} TFLOP/s), unfused {t_u:.4f} ms "
                f"({f / t_u / 1e9:.1f} TFLOP/s), unfused/fused {t_u / t_f:.3f}; same code unfused {t_s:.4f} ms "
                f"({t_s / t_f:.3f}x fused)")
            del a, w, a_full, out
            torch.cuda.empty_cache()
    line = {
        "metric": AG_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, **cfg.as_dict(), "algorithmic_flops": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "kernel": "mkag::ag_gemm_kernel",
                     "shader_clock_ghz": round(clock, 3) if clock else None},
        "unfused_baseline": {"what": "device copy of the shards into A_full, then torch.matmul (hipBLASLt)",
                             "ms": round(ms_unf, 4), "unfused_over_fused": round(ms_unf / ms, 3)},
        "unfused_same_code": {"what": "the gather phase, then the GEMM phase of the same kernel (two launches)",
                              "ms": round(ms_same, 4), "over_fused": round(ms_same / ms, 3),
                              "gemm_phase_ms": round(ms_gemm, 4)},
        "split_sweep": {"ms": split, "best_fixed": best, "adaptive_over_best": round(split["adaptive"] / split[best], 3),
                        "adaptive_paper_over_best": round(split["adaptive_paper"] / split[best], 3)},
        "staging": {k: st[k] for k in ("grid_wgs", "staging_tasks", "assist_tasks", "max_staging_wgs")},
    }
    if sweep:
        line["size_sweep"] = sweep
    print(json.dumps(line), flush=True)


PROBE_MODES = (
    (2, "MFMA + ds_read_b128, random bf16"),
    (0, "MFMA, random bf16 from registers"),
    (1, "MFMA + ds_read_b128, constant data"),
    (3, "MFMA + ds_read_b128, random bf16, + exp2 and FMA per MFMA"),
)


def run_probes(rounds=3):
    """Runs libmkra_probes.so: MFMA streams (8 waves per CU, about 0.2 s per launch, the
    modes in turn, `rounds` times; median per mode) and the v_exp_f32 / v_fma_f32 issue
    rates. Returns markdown."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "overlap_attention_amd", "libmkra_probes.so"))
    for fn in (lib.mkp_mfma_stream, lib.mkp_valu_rate):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
        fn.restype = ctypes.c_int
    lib.mkp_lds_rate.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.mkp_lds_rate.restype = ctypes.c_int
    lib.mkp_coexec.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.mkp_coexec.restype = ctypes.c_int

    def call(fn, mode, iters):
        res = (ctypes.c_double * 4)()
        if fn(mode, iters, res) != 0:
            raise RuntimeError("probe failed (mode %d)" % mode)
        return list(res)

    rows = {m: [] for m, _ in PROBE_MODES}
    for r in range(rounds):
        for m, name in PROBE_MODES:
            rows[m].append(call(lib.mkp_mfma_stream, m, 150000))
            log(f"[probes] round {r} mode {m}: {rows[m][-1][2]:.0f} TFLOP/s at {rows[m][-1][1]:.3f} GHz")
    out = ["| MFMA stream (v_mfma_f32_32x32x16_bf16, 8 waves per CU) | ms | shader clock GHz | TFLOP/s | "
           "% of 2.4 GHz peak | % of peak at its clock |", "|---|---:|---:|---:|---:|---:|"]
    for m, name in PROBE_MODES:
        ms, ghz, tf, _ = sorted(rows[m], key=lambda x: x[2])[len(rows[m]) // 2]
        out.append(f"| {name} | {ms:.1f} | {ghz:.3f} | {tf:.0f} | {100 * tf / PEAK_BF16_TFLOPS:.1f} | "
                   f"{100 * tf / (PEAK_BF16_TFLOPS * ghz / PEAK_CLOCK_GHZ):.1f} |")
    out += ["", "| vector op (8 independent chains per lane, 8 waves per CU) | ms | shader clock GHz | "
            "lane-ops per clock per CU |", "|---|---:|---:|---:|"]
    for m, name in ((0, "v_exp_f32"), (1, "v_fma_f32")):
        ms, ghz, rate, _ = call(lib.mkp_valu_rate, m, 200000)
        log(f"[probes] {name}: {rate:.1f} lane-ops/clk/CU")
        out.append(f"| {name} | {ms:.1f} | {ghz:.3f} | {rate:.1f} |")
    out += ["", "| LDS reads (ds_read_b128, no bank conflicts, 8 waves per CU) | ms | shader clock GHz | "
            "bytes per clock per CU |", "|---|---:|---:|---:|"]
    lds = []
    for r in range(rounds):
        res = (ctypes.c_double * 4)()
        if lib.mkp_lds_rate(400000, res) != 0:
            raise RuntimeError("probe failed (LDS rate)")
        lds.append(list(res))
        log(f"[probes] round {r} LDS reads: {res[2]:.1f} bytes/clk/CU at {res[1]:.3f} GHz")
    ms, ghz, rate, _ = sorted(lds, key=lambda x: x[2])[len(lds) // 2]
    out.append(f"| ds_read_b128 | {ms:.1f} | {ghz:.3f} | {rate:.1f} |")
    out += ["", "| two waves per SIMD: first runs MFMAs (32 per iteration, each with a 1 KiB ds_read_b128), "
            "second one block's softmax per iteration | ms | MFMA wave cycles per iteration | "
            "softmax wave cycles per iteration |", "|---|---:|---:|---:|"]
    for mode, name in ((0, "MFMA waves alone"), (1, "softmax waves alone"), (2, "both at once")):
        runs = []
        for r in range(rounds):
            res = (ctypes.c_double * 4)()
            if lib.mkp_coexec(mode, 20000, res) != 0:
                raise RuntimeError("probe failed (co-execution mode %d)" % mode)
            runs.append(list(res))
            log(f"[probes] round {r} co-execution {name}: MFMA {res[1]:.0f}, softmax {res[2]:.0f} cycles per iteration")
        ms, cm, cs, _ = sorted(runs, key=lambda x: x[0])[len(runs) // 2]
        out.append(f"| {name} | {ms:.1f} | {cm:.0f} | {cs:.0f} |")
    return "\n".join(out)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "the host CPU"


def oracle_timed(cfg, q, kv, rows, progress=False):
    """One timed pass of the fp64 oracle over `rows` (None: every row) of a workload,
    all heads: the oracle's own function, called once per KV head (a complete problem
    of its own), the KV heads spread over the cores of this process's affinity mask,
    BLAS at one thread each. Returns (seconds, algorithmic FLOPs covered, cores)."""
    import numpy as np

    import oracle
    from ring_inputs import to_f64
    from tests.parity import oracle_rows

    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, cfg.hkv))
    q64, kv64 = to_f64(q), to_f64(kv)
    rr = np.arange(cfg.lq) if rows is None else np.asarray(rows)
    t0 = time.perf_counter()
    oracle_rows(oracle, q64, kv64, cfg.rank, cfg.causal, cfg.gqa_ratio, rr, workers=workers, progress=progress)
    dt = time.perf_counter() - t0
    if cfg.causal:
        pairs = int(sum(cfg.rank * cfg.lk + int(r) + 1 for r in rr))
    else:
        pairs = len(rr) * cfg.n_chunks * cfg.lk
    return dt, 4 * cfg.d * cfg.hq * pairs, workers


def cpu_baseline(cfg, q, kv, budget_rows):
    """The fp64 oracle on the host cores, on the same workload: every query row when
    `budget_rows` is 0 or at least the chunk's rows (the default; about 10 s for the
    64K-token workload), else `budget_rows` rows spread evenly over the chunk; all
    heads, all keys."""
    import numpy as np

    if budget_rows <= 0 or budget_rows >= cfg.lq:
        rows, what = None, f"every query row ({cfg.lq})"
    else:
        rows = np.linspace(0, cfg.lq - 1, budget_rows).astype(np.int64)
        what = f"{len(rows)} of {cfg.lq} query rows (evenly spaced)"
    dt, flops, workers = oracle_timed(cfg, q, kv, rows)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{what}, all {cfg.hq} heads, all visible keys; "
                  f"{dt:.1f} s on {workers} threads (one KV head per call, BLAS at one thread each; "
                  f"{len(os.sched_getaffinity(0))} cores in the affinity mask) of {_cpu_model()}; fp64 NumPy, "
                  f"dense over masked keys too (FLOPs counted for visible pairs only)",
    }


def cpu_all_workloads():
    """One timed oracle pass per workload (every query row, all heads), on the host
    cores. Returns markdown."""
    from ring_inputs import CONFIGS, make_inputs

    lines = [f"Host: {_cpu_model()}, {len(os.sched_getaffinity(0))} cores in the affinity mask.", "",
             "| workload | rows | seconds | threads | algorithmic GFLOP/s |", "|---|---:|---:|---:|---:|"]
    for i, cfg in enumerate(CONFIGS):
        q, kv = make_inputs(cfg, seed=i)
        dt, flops, workers = oracle_timed(cfg, q, kv, None, progress=True)
        log(f"[cpu] {cfg.name}: {dt:.1f} s, {flops / dt / 1e9:.1f} GFLOP/s on {workers} threads")
        lines.append(f"| {cfg.name} | {cfg.lq} | {dt:.2f} | {workers} | {flops / dt / 1e9:.1f} |")
        del q, kv
    # The AllGather+GEMM oracle: one float64 product of the gathered shards, BLAS over
    # the affinity mask's cores.
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from ag_inputs import AG_CONFIGS, make_ag_inputs
    lines += ["", "| AllGather+GEMM workload | gathered rows | seconds | threads | algorithmic GFLOP/s |",
              "|---|---:|---:|---:|---:|"]
    cores = len(os.sched_getaffinity(0))
    for cfg in AG_CONFIGS:
        a, w = make_ag_inputs(cfg, seed=1)
        a64, w64 = a.double().numpy(), w.double().numpy()
        with threadpool_limits(cores):
            t0 = time.perf_counter()
            oracle.allgather_gemm_reference(a64, w64, cfg.rank)
            dt = time.perf_counter() - t0
        flops = 2.0 * cfg.m * cfg.n_out * cfg.k
        log(f"[cpu] {cfg.name}: {dt:.1f} s, {flops / dt / 1e9:.1f} GFLOP/s on {cores} threads")
        lines.append(f"| {cfg.name} | {cfg.m} | {dt:.2f} | {cores} | {flops / dt / 1e9:.1f} |")
        del a, w, a64, w64
    return "\n".join(lines)


def kernel_stats_from(trace_dir, warmup, steps, kernel="ring_attn_kernel"):
    """Durations of the timed dispatches of the ring kernel in a rocprofv3
    --kernel-trace run of `bench.py --steps K --warmup W`: the ring kernel's dispatches
    in order are W warm-ups, then the K timed ones, then the statistics call; only the
    K timed ones are summarised. Returns markdown."""
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)):
        rows += [r for r in csv.DictReader(open(f)) if kernel in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no {kernel} dispatches in a *kernel_trace.csv under {trace_dir}")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6 for r in rows]
    if len(dur) < warmup + steps:
        raise SystemExit(f"{len(dur)} dispatches, expected at least {warmup + steps}")
    timed = dur[warmup:warmup + steps]
    st = sorted(timed)
    med = statistics.median(timed)
    span = (int(rows[warmup + steps - 1]["End_Timestamp"]) - int(rows[warmup]["Start_Timestamp"])) * 1e-6
    return "\n".join([
        f"Kernel `{rows[0]['Kernel_Name']}`: {len(dur)} dispatches; dispatches {warmup}..{warmup + steps - 1} "
        f"are the {steps} timed launches.", "",
        "| timed dispatches | median ms | mean ms | min ms | max ms | first start to last end, ms per launch |",
        "|---:|---:|---:|---:|---:|---:|",
        f"| {steps} | {med:.4f} | {sum(timed) / steps:.4f} | {st[0]:.4f} | {st[-1]:.4f} | {span / steps:.4f} |",
        "", "All dispatches (ms): " + ", ".join(f"{d:.3f}" for d in dur)])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="name of a workload in ring_inputs.CONFIGS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="query rows of the CPU oracle baseline (0: every row of the workload)")
    ap.add_argument("--repeats", type=int, default=5, help="groups the timed launches are split into (median, min)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time fixed staging splits {1..64} against the adaptive split (Fig. 3's metric)")
    ap.add_argument("--size-sweep", action="store_true",
                    help="also run the split sweep over total sequence sizes 6K..192K (16 ranks, rank 15)")
    ap.add_argument("--unfused", action="store_true",
                    help="also time the unfused two-stream baseline against the fused kernel over sequence sizes "
                         "6K..192K (16 ranks, rank 15)")
    ap.add_argument("--verify", action="store_true", help="check sampled rows against the oracle (stderr)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (3 times), the known-size "
                         "reference that scales the HBM byte counters")
    ap.add_argument("--traffic-from", default=None,
                    help="no GPU: turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs (DIR/fetch, DIR/write) into "
                         "profiles/traffic_<workload>.json")
    ap.add_argument("--probes", action="store_true",
                    help="run the MFMA-stream, vector-ALU, LDS-read and co-execution probes instead of the benchmark; prints markdown")
    ap.add_argument("--ag", action="store_true",
                    help="benchmark one rank's AllGather+GEMM instead (fused kernel, unfused copy + library GEMM, "
                         "split sweep); prints its own JSON line")
    ap.add_argument("--ag-workload", default=None, help="name of a workload in ag_inputs.AG_CONFIGS")
    ap.add_argument("--ag-sweep", action="store_true", help="with --ag: also sweep the gathered size 4K..32K rows")
    ap.add_argument("--cpu-all", action="store_true",
                    help="no GPU: one timed oracle pass (every row) per workload on the host cores; prints markdown")
    ap.add_argument("--kernel-stats-from", default=None,
                    help="no GPU: summarise the timed dispatches (after --warmup, --steps of them) of a rocprofv3 "
                         "--kernel-trace run under DIR; prints markdown")
    args = ap.parse_args()
    if args.probes:
        print(run_probes(), flush=True)
        return
    if args.cpu_all:
        print(cpu_all_workloads(), flush=True)
        return
    if args.ag:
        if args.gpus != 1:
            print("bench.py runs on one GPU only: this library has no multi-GPU path (use --gpus 1).", file=sys.stderr)
            sys.exit(2)
        run_ag(args)
        return
    if args.kernel_stats_from:
        print(kernel_stats_from(args.kernel_stats_from, args.warmup, args.steps), flush=True)
        return
    if args.traffic_from:
        from ring_inputs import CONFIG_BY_NAME, SEQ64K

        cfg = CONFIG_BY_NAME[args.workload] if args.workload else SEQ64K
        write_traffic(cfg, args.traffic_from, args.copy_calibration_mib or 1024)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import overlap_attention_amd as mk
    from ring_inputs import CONFIG_BY_NAME, CONFIGS, SEQ64K, make_inputs

    cfg = CONFIG_BY_NAME[args.workload] if args.workload else SEQ64K
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    log(f"[bench] workload {cfg.name}: generating inputs")
    q, kv = make_inputs(cfg, seed=CONFIGS.index(cfg) if cfg in CONFIGS else 0)
    qg, kvg = q.cuda(), kv.cuda()
    out = torch.empty_like(qg)
    lse = torch.empty((cfg.hq, cfg.lq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(opts=None):
        if opts is None:
            mk.mk_ring_attn_fwd(qg, kvg, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, out, lse, stream=stream)
        else:
            mk.mk_ring_attn_fwd_ex(qg, kvg, cfg.n_chunks, cfg.rank, cfg.causal, cfg.gqa_ratio, out, lse,
                                   stream=stream, opts=opts)

    def timed(k, opts=None, groups=1):
        """Mean ms per launch over k launches back to back on the stream, and the
        per-launch time of each of `groups` consecutive groups of them (HIP events
        recorded on the same stream between the groups)."""
        groups = max(1, min(groups, k))
        sizes = [k // groups + (1 if i < k % groups else 0) for i in range(groups)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for g, n in enumerate(sizes):
            for _ in range(n):
                step(opts)
            evs[g + 1].record(stream)
        torch.cuda.synchronize()
        per_group = [evs[g].elapsed_time(evs[g + 1]) / n for g, n in enumerate(sizes)]
        return evs[0].elapsed_time(evs[-1]) / k, per_group

    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy calibration: 3 x {args.copy_calibration_mib} MiB")
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mk.mk_ring_attn_status()
    log(f"[bench] timing {args.steps} launches")
    t_host0 = time.perf_counter()
    ms, per_group = timed(args.steps, groups=args.repeats)
    t_host = time.perf_counter() - t_host0
    ms_median = statistics.median(per_group)
    ms_min = min(per_group)
    mk.mk_ring_attn_status()
    flops = algorithmic_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/launch, {tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of peak); "
        f"groups of {args.steps // max(1, args.repeats)}: median {ms_median:.3f} ms, min {ms_min:.3f} ms; "
        f"host wall {t_host:.3f} s")

    stats = mk.ring_attn_fwd(qg, kvg, cfg.rank, cfg.causal, cfg.gqa_ratio, want_stats=True)[2]
    log(f"[bench] stats {stats}")

    if args.verify:
        import oracle
        from ring_inputs import to_f64
        from tests.parity import compare, fmt, sample_rows

        rows = sample_rows(cfg.lq, n_random=8, seed=1)
        ro, rl = oracle.ring_attention_rows(to_f64(q), to_f64(kv), cfg.rank, cfg.causal, cfg.gqa_ratio, rows)
        rep = compare(to_f64(out[rows]), lse[:, rows].double().cpu().numpy(), ro, rl)
        log(f"[bench] verify: {fmt(rep)}")

    sweep = None
    if args.sweep:
        sweep = split_sweep(mk, timed, max(3, args.steps // 3))
        log("[bench] sweep (ms/launch, latency / best fixed): " +
            ", ".join(f"{k}={v:.3f} ({v / sweep['best_fixed_ms']:.2f}x)" for k, v in sweep["ms"].items()))
    size_sweep = None
    if args.size_sweep:
        size_sweep = run_size_sweep(torch, mk, make_inputs, stream)
    unfused_sweep = None
    if args.unfused:
        unfused_sweep = run_unfused_sweep(torch, mk, make_inputs, stream)

    traffic = stored_traffic(cfg.name)
    # Average shader clock over every workgroup's lifetime (s_memtime cycles against
    # 100 MHz ticks), and the MFMA peak scaled to it: the fraction the schedule
    # reaches at the clock the chip actually ran, next to the one at 2.4 GHz.
    clock_ghz = (stats["wg_cycles"] / stats["wg_ticks"] * 0.1) if stats["wg_ticks"] > 0 else None
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 QK / fp16 PV",
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "rank": cfg.rank,
            "n_chunks": cfg.n_chunks,
            "lq": cfg.lq,
            "lk": cfg.lk,
            "hq": cfg.hq,
            "hkv": cfg.hkv,
            "head_dim": cfg.d,
            "causal": cfg.causal,
            "algorithmic_flops": flops,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_bytes": algorithmic_bytes(cfg),
            "kernel": "mkra::ring_attn_kernel<%d>" % cfg.d,
            "shader_clock_ghz": round(clock_ghz, 3) if clock_ghz else None,
            "frac_at_shader_clock": (round(tflops / (PEAK_BF16_TFLOPS * clock_ghz / PEAK_CLOCK_GHZ), 4)
                                     if clock_ghz else None),
        },
        "timing": {"groups": args.repeats, "median_ms_per_step": round(ms_median, 4),
                   "min_ms_per_step": round(ms_min, 4)},
        "staging": staging_summary(cfg, stats, ms),
    }
    if sweep is not None:
        line["split_sweep"] = sweep
    if size_sweep is not None:
        line["size_sweep"] = size_sweep
    if unfused_sweep is not None:
        line["unfused_sweep"] = unfused_sweep
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows or cfg.lq} rows")
        line["cpu_baseline"] = cpu_baseline(cfg, q, kv, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
