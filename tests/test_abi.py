"""The C-ABI library loads, exports every entry point include/*.h declares, and
rejects bad arguments on the host before touching a GPU. Runs without a GPU."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import overlap_attention_amd as mk
from overlap_attention_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(mk_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_header_lists_the_entry_points():
    names = declared_functions()
    assert "mk_ring_attn_fwd" in names and "mk_ring_attn_fwd_ex" in names and "mk_allgather_gemm" in names
    assert set(names) == set(B._PROTOTYPES), names


def test_library_exports_every_declared_symbol():
    lib = mk.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mk.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    # Nothing else leaks into the ABI.
    assert {s for s in exported if not s.startswith("_")} == set(declared_functions())


def test_probe_library_exports_its_four_entry_points():
    # The measurement probes (bench.py --probes) live in a library of their own, so the
    # ring-attention library's ABI stays exactly what include/mkra.h declares.
    path = os.path.join(os.path.dirname(mk.LIB_PATH), "libmkra_probes.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = {s for s in re.findall(r"\bT\s+(\w+)$", out, flags=re.M) if not s.startswith("_")}
    assert exported == {"mkp_mfma_stream", "mkp_valu_rate", "mkp_lds_rate", "mkp_coexec"}, exported
    lib = ctypes.CDLL(path)
    res = (ctypes.c_double * 4)()
    # Bad arguments are refused before any device call.
    assert lib.mkp_mfma_stream(7, 10, res) == 1
    assert lib.mkp_valu_rate(0, 0, res) == 1
    assert lib.mkp_lds_rate(0, res) == 1
    assert lib.mkp_coexec(3, 10, res) == 1


def test_abi_version():
    assert mk.mk_abi_version() == 2


def test_struct_layouts_match_the_header():
    """sizeof/offsetof of the C structs, compiled from the header with gcc, equal the
    ctypes mirror's."""
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "mkag.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(mk_tensor), sizeof(mk_ring_attn_opts), sizeof(mk_ring_attn_stats),
         sizeof(mk_trace_record));
  printf("%zu %zu %zu %zu %zu %zu\n", offsetof(mk_ring_attn_opts, spin_timeout_us), offsetof(mk_ring_attn_opts, trace),
         offsetof(mk_ring_attn_stats, compute_busy_ticks), offsetof(mk_ring_attn_stats, trace_records),
         offsetof(mk_ring_attn_opts, debug_flags), offsetof(mk_ring_attn_stats, debug_mismatches));
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(mk_ag_gemm_opts), sizeof(mk_ag_gemm_stats),
         offsetof(mk_ag_gemm_opts, spin_timeout_us), offsetof(mk_ag_gemm_stats, compute_busy_ticks),
         offsetof(mk_ag_gemm_stats, wg_ticks), offsetof(mk_ag_gemm_opts, disable_staging));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(prog)
        r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                            "-I/opt/rocm/include", c, "-o", exe], capture_output=True, text=True)
        if r.returncode != 0:
            pytest.skip("no C compiler for the layout check: " + r.stderr[-300:])
        sizes, offs, ag = subprocess.run([exe], capture_output=True, text=True).stdout.split("\n")[:3]
    assert [int(x) for x in sizes.split()] == [ctypes.sizeof(B.mk_tensor), ctypes.sizeof(B.mk_ring_attn_opts),
                                               ctypes.sizeof(B.mk_ring_attn_stats),
                                               ctypes.sizeof(B.mk_trace_record)]
    assert [int(x) for x in offs.split()] == [B.mk_ring_attn_opts.spin_timeout_us.offset,
                                              B.mk_ring_attn_opts.trace.offset,
                                              B.mk_ring_attn_stats.compute_busy_ticks.offset,
                                              B.mk_ring_attn_stats.trace_records.offset,
                                              B.mk_ring_attn_opts.debug_flags.offset,
                                              B.mk_ring_attn_stats.debug_mismatches.offset]
    assert [int(x) for x in ag.split()] == [ctypes.sizeof(B.mk_ag_gemm_opts), ctypes.sizeof(B.mk_ag_gemm_stats),
                                            B.mk_ag_gemm_opts.spin_timeout_us.offset,
                                            B.mk_ag_gemm_stats.compute_busy_ticks.offset,
                                            B.mk_ag_gemm_stats.wg_ticks.offset,
                                            B.mk_ag_gemm_opts.disable_staging.offset]


def test_default_opts():
    o = mk.default_opts()
    assert o.split_mode == mk.MK_SPLIT_ADAPTIVE and o.grid_wgs == 0 and o.disable_staging == 0
    assert o.parallel_steps == 0  # automatic: parallel step groups for launches with few units
    assert o.stage_pieces == 0  # automatic: staging pieces per tile from the problem's size


# ---------------------------------------------------------------- host validation

FAKE = 1 << 32  # aligned, never dereferenced: validation fails before any HIP call


def desc(shape, dtype=B.MK_BF16, ptr=FAKE, strides=None):
    d = B.mk_tensor()
    d.data = ptr
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def call(q, kv, n, rank, causal, g, out, lse, opts=None):
    lib = mk.load_library()
    byref = lambda x: ctypes.byref(x) if x is not None else None  # noqa: E731
    if opts is None:
        return lib.mk_ring_attn_fwd(byref(q), byref(kv), n, rank, causal, g, byref(out), byref(lse), None)
    return lib.mk_ring_attn_fwd_ex(byref(q), byref(kv), n, rank, causal, g, byref(out), byref(lse), None,
                                   ctypes.byref(opts), None)


def good(lq=256, lk=256, hq=8, hkv=2, d=128, n=4):
    base = FAKE
    q = desc([lq, hq, d], ptr=base)
    kv = desc([n, 2, lk, hkv, d], ptr=base + (1 << 30))
    out = desc([lq, hq, d], ptr=base + (2 << 30))
    lse = desc([hq, lq], dtype=B.MK_F32, ptr=base + (3 << 30))
    return q, kv, out, lse


CASES = {
    "null_q": lambda q, kv, o, l: (None, kv, 4, 1, 1, 4, o, l),
    "null_out": lambda q, kv, o, l: (q, kv, 4, 1, 1, 4, None, l),
    "q_dtype": lambda q, kv, o, l: (desc([256, 8, 128], dtype=B.MK_F32), kv, 4, 1, 1, 4, o, l),
    "lse_dtype": lambda q, kv, o, l: (q, kv, 4, 1, 1, 4, o, desc([8, 256], dtype=B.MK_BF16, ptr=FAKE + (3 << 30))),
    "rank_too_big": lambda q, kv, o, l: (q, kv, 4, 4, 1, 4, o, l),
    "rank_negative": lambda q, kv, o, l: (q, kv, 4, -1, 1, 4, o, l),
    "n_chunks_mismatch": lambda q, kv, o, l: (q, kv, 3, 1, 1, 4, o, l),
    "gqa_mismatch": lambda q, kv, o, l: (q, kv, 4, 1, 1, 2, o, l),
    "gqa_zero": lambda q, kv, o, l: (q, kv, 4, 1, 1, 0, o, l),
    "causal_lq_ne_lk": lambda q, kv, o, l: (desc([128, 8, 128]), kv, 4, 1, 1, 4,
                                            desc([128, 8, 128], ptr=FAKE + (2 << 30)),
                                            desc([8, 128], dtype=B.MK_F32, ptr=FAKE + (3 << 30))),
    "non_contiguous_q": lambda q, kv, o, l: (desc([256, 8, 128], strides=[2048, 128, 2]), kv, 4, 1, 1, 4, o, l),
    "misaligned_q": lambda q, kv, o, l: (desc([256, 8, 128], ptr=FAKE + 2), kv, 4, 1, 1, 4, o, l),
    "out_shape": lambda q, kv, o, l: (q, kv, 4, 1, 1, 4, desc([256, 8, 64], ptr=FAKE + (2 << 30)), l),
    "lse_shape": lambda q, kv, o, l: (q, kv, 4, 1, 1, 4, o, desc([256, 8], dtype=B.MK_F32, ptr=FAKE + (3 << 30))),
    "out_overlaps_q": lambda q, kv, o, l: (q, kv, 4, 1, 1, 4, desc([256, 8, 128], ptr=FAKE + 4096), l),
    "kv_second_dim": lambda q, kv, o, l: (q, desc([4, 3, 256, 2, 128], ptr=FAKE + (1 << 30)), 4, 1, 1, 4, o, l),
    "head_dim_mismatch": lambda q, kv, o, l: (q, desc([4, 2, 256, 2, 64], ptr=FAKE + (1 << 30)), 4, 1, 1, 4, o, l),
    "no_keys": lambda q, kv, o, l: (desc([256, 8, 128]), desc([4, 2, 0, 2, 128], ptr=FAKE + (1 << 30)), 4, 1, 0,
                                    4, o, l),
    "null_data": lambda q, kv, o, l: (desc([256, 8, 128], ptr=None), kv, 4, 1, 1, 4, o, l),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_invalid_arguments_rejected_on_host(name):
    q, kv, o, l = good()
    args = CASES[name](q, kv, o, l)
    assert call(*args) == mk.MK_E_INVAL, name
    assert mk.load_library().mk_last_error().decode() != ""


def test_unsupported_head_dim():
    q, kv, o, l = good(d=96)
    assert call(q, kv, 4, 1, 1, 4, o, l) == mk.MK_E_UNSUPPORTED
    assert b"head_dim" in mk.load_library().mk_last_error()


def test_negative_option_rejected():
    q, kv, o, l = good()
    opts = mk.default_opts(grid_wgs=-1)
    assert call(q, kv, 4, 1, 1, 4, o, l, opts) == mk.MK_E_INVAL
    opts = mk.default_opts(split_mode=7)
    assert call(q, kv, 4, 1, 1, 4, o, l, opts) == mk.MK_E_INVAL
    for ps in (-2, 2):
        assert call(q, kv, 4, 1, 1, 4, o, l, mk.default_opts(parallel_steps=ps)) == mk.MK_E_INVAL
        assert b"parallel_steps" in mk.load_library().mk_last_error()
    assert call(q, kv, 4, 1, 1, 4, o, l, mk.default_opts(stage_pieces=-1)) == mk.MK_E_INVAL
    assert b"stage_pieces" in mk.load_library().mk_last_error()


def test_empty_query_is_a_noop():
    q, kv, o, l = good(lq=0, lk=0)
    # causal with Lq == Lk == 0, nothing to compute: returns before any HIP call.
    assert call(desc([0, 8, 128], ptr=None), desc([4, 2, 0, 2, 128], ptr=None), 4, 1, 1, 4,
                desc([0, 8, 128], ptr=None), desc([8, 0], dtype=B.MK_F32, ptr=None)) == mk.MK_OK


def test_missing_library_fails_loudly(tmp_path):
    saved = B._lib
    B._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            B.load_library(str(tmp_path / "nope.so"))
    finally:
        B._lib = saved


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "overlap_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, flags=re.M), f
                assert "ring_attention_reference" not in src and "allgather_gemm_reference" not in src, f
    oracle_dir = os.path.join(ROOT, "oracle")
    for f in os.listdir(oracle_dir):
        if f.endswith(".py"):
            src = open(os.path.join(oracle_dir, f)).read()
            assert "overlap_attention_amd" not in src and "ring_inputs" not in src and "ag_inputs" not in src, f
