"""Host logic of bench.py that turns a run into the numbers it reports (no GPU): the
algorithmic FLOP count behind TFLOP/s and the roofline, the HBM traffic computed from
rocprofv3 counter CSVs, and the selection of the timed dispatches from a kernel trace.
The profiler files are small synthetic ones with the columns rocprofv3 writes."""

import csv
import json
import os

import pytest

import bench
import oracle
from ring_inputs import CONFIGS, RingConfig


def visible_pairs_brute_force(cfg):
    """Visible (query, key) pairs counted one by one: query i of rank r sits at global
    position r*L + i; causal attention sees keys at positions up to its own."""
    n = 0
    for i in range(cfg.lq):
        qpos = cfg.rank * cfg.lq + i
        for c in range(cfg.n_chunks):
            for j in range(cfg.lk):
                if not cfg.causal or c * cfg.lk + j <= qpos:
                    n += 1
    return n


@pytest.mark.parametrize("cfg", [
    RingConfig("t1", rank=2, n_chunks=4, lq=5, lk=5, hq=3, hkv=1, d=64, causal=True),
    RingConfig("t2", rank=0, n_chunks=3, lq=4, lk=4, hq=2, hkv=2, d=128, causal=True),
    RingConfig("t3", rank=1, n_chunks=3, lq=3, lk=6, hq=4, hkv=2, d=64, causal=False),
], ids=lambda c: c.name)
def test_algorithmic_flops_count_visible_pairs(cfg):
    assert bench.algorithmic_flops(cfg) == 4 * cfg.d * cfg.hq * visible_pairs_brute_force(cfg)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_algorithmic_flops_agree_with_the_oracle_count(cfg):
    assert bench.algorithmic_flops(cfg) == oracle.attention_flops(cfg.lq, cfg.lk, cfg.n_chunks, cfg.rank, cfg.causal,
                                                                   cfg.hq, cfg.d)


def test_headline_flops():
    # Rank 15 of a 64K-token causal ring: 15 full 4096 x 4096 chunks and one triangle
    # with its diagonal, 32 heads, 4 * 128 FLOPs per visible pair.
    cfg = next(c for c in CONFIGS if c.name.startswith("seq64k"))
    assert bench.algorithmic_flops(cfg) == 4 * 128 * 32 * (15 * 4096 * 4096 + 4096 * 4097 // 2) == 4260641112064


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def counter_rows(counter, ring_values, copy_values):
    rows = []
    for i, v in enumerate(ring_values):
        rows.append({"Dispatch_Id": 10 + i, "Kernel_Name": "void mkra::ring_attn_kernel<128>(mkra::KernelArgs)",
                     "Grid_Size": 131072, "Counter_Name": counter, "Counter_Value": v})
    # Two copies: a small one and the calibration copy (the largest grid).
    rows.append({"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 4096,
                 "Counter_Name": counter, "Counter_Value": 7})
    for i, v in enumerate(copy_values):
        rows.append({"Dispatch_Id": 2 + i, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 1 << 20,
                     "Counter_Name": counter, "Counter_Value": v})
    return rows


def test_traffic_from_counter_csvs(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0123456789abcdef")
    os.makedirs(tmp_path / "profiles")
    pmc = tmp_path / "pmc"
    mib = 64
    n32 = mib * 1024 * 1024 // 32  # 32-byte requests of a copy of `mib` MiB
    # The first ring dispatch is left out (median over the later ones).
    write_csv(str(pmc / "dram" / "run_counter_collection.csv"),
              counter_rows("TCC_EA0_RDREQ_DRAM_32B_sum", [999, 100, 300, 200], [n32, n32])
              + counter_rows("TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", [5, 40, 60, 50], [n32, n32]))
    # FETCH_SIZE reads half the copy's bytes, so it is scaled by 2.
    write_csv(str(pmc / "fetch" / "run_counter_collection.csv"),
              counter_rows("FETCH_SIZE", [1, 10, 30, 20], [mib * 512, mib * 512]))
    cfg = next(c for c in CONFIGS if c.name.startswith("seq64k"))
    bench.write_traffic(cfg, str(pmc), mib)
    out = json.load(open(tmp_path / "profiles" / f"traffic_{cfg.name}.json"))
    assert out["kernel_sha"] == "0123456789abcdef"
    assert out["hbm_bytes_per_launch"] == 32 * (200 + 50)
    assert out["counters"]["dram_32b"]["read"]["copy_over_moved"] == 1.0
    assert out["counters"]["FETCH_SIZE"]["scale"] == 2.0
    assert out["counters"]["FETCH_SIZE"]["bytes_per_launch"] == 20 * 1024 * 2.0
    assert out["algorithmic_bytes"] == bench.algorithmic_bytes(cfg)
    # The stored figure is reported only while the kernel source is the one measured.
    assert bench.stored_traffic(cfg.name) == 32 * 250
    monkeypatch.setattr(bench, "kernel_hash", lambda: "fedcba9876543210")
    assert bench.stored_traffic(cfg.name) is None


def test_kernel_stats_take_the_timed_dispatches(tmp_path):
    rows, t = [], 1_000_000
    durations = [9.0, 8.0] + [3.0, 5.0, 4.0] + [7.0]  # 2 warm-ups, 3 timed, the statistics call
    for i, d in enumerate(durations):
        rows.append({"Kernel_Name": "void mkra::ring_attn_kernel<128>(mkra::KernelArgs)", "Start_Timestamp": t,
                     "End_Timestamp": t + int(d * 1e6)})
        rows.append({"Kernel_Name": "__amd_rocclr_fillBufferAligned", "Start_Timestamp": t + int(d * 1e6) + 10,
                     "End_Timestamp": t + int(d * 1e6) + 20})
        t += int(d * 1e6) + 1000
    write_csv(str(tmp_path / "kt" / "run_kernel_trace.csv"), rows)
    md = bench.kernel_stats_from(str(tmp_path / "kt"), 2, 3)
    line = next(l for l in md.splitlines() if l.startswith("| 3 |"))
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert [float(c) for c in cells[1:5]] == [4.0, 4.0, 3.0, 5.0]  # median, mean, min, max of the timed three
    with pytest.raises(SystemExit):
        bench.kernel_stats_from(str(tmp_path / "kt"), 5, 3)  # fewer dispatches than warm-ups + steps
