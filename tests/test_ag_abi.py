"""Host-side validation of the AllGather+GEMM entry points (include/mkag.h): bad
arguments are refused before any HIP call. Runs without a GPU."""

import ctypes

import pytest

import overlap_attention_amd as mk
from overlap_attention_amd import _binding as B
from tests.test_abi import FAKE, desc


def call(a, n, rank, w, af, c, opts=None):
    lib = mk.load_library()
    byref = lambda x: ctypes.byref(x) if x is not None else None  # noqa: E731
    if opts is None:
        return lib.mk_allgather_gemm(byref(a), n, rank, byref(w), byref(af), byref(c), None)
    return lib.mk_allgather_gemm_ex(byref(a), n, rank, byref(w), byref(af), byref(c), None, ctypes.byref(opts), None)


def good(n=4, m=256, k=512, no=1024):
    return (desc([n, m, k], ptr=FAKE), desc([no, k], ptr=FAKE + (1 << 30)), desc([n * m, k], ptr=FAKE + (2 << 30)),
            desc([n * m, no], ptr=FAKE + (3 << 30)))


CASES = {
    "null_a": lambda a, w, f, c: (None, 4, 1, w, f, c),
    "null_c": lambda a, w, f, c: (a, 4, 1, w, f, None),
    "a_dtype": lambda a, w, f, c: (desc([4, 256, 512], dtype=B.MK_F32), 4, 1, w, f, c),
    "rank_too_big": lambda a, w, f, c: (a, 4, 4, w, f, c),
    "rank_negative": lambda a, w, f, c: (a, 4, -1, w, f, c),
    "n_ranks_mismatch": lambda a, w, f, c: (a, 3, 1, w, f, c),
    "w_k_mismatch": lambda a, w, f, c: (a, 4, 1, desc([1024, 256], ptr=FAKE + (1 << 30)), f, c),
    "a_full_shape": lambda a, w, f, c: (a, 4, 1, w, desc([1000, 512], ptr=FAKE + (2 << 30)), c),
    "c_shape": lambda a, w, f, c: (a, 4, 1, w, f, desc([1024, 1000], ptr=FAKE + (3 << 30))),
    "c_overlaps_a": lambda a, w, f, c: (a, 4, 1, w, f, desc([1024, 1024], ptr=FAKE + 4096)),
    "a_full_overlaps_w": lambda a, w, f, c: (a, 4, 1, w, desc([1024, 512], ptr=FAKE + (1 << 30) + 64), c),
    "non_contiguous_w": lambda a, w, f, c: (a, 4, 1, desc([1024, 512], ptr=FAKE + (1 << 30), strides=[1024, 1]), f, c),
    "misaligned_a": lambda a, w, f, c: (desc([4, 256, 512], ptr=FAKE + 2), 4, 1, w, f, c),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_invalid_arguments_rejected_on_host(name):
    args = CASES[name](*good())
    assert call(*args) == mk.MK_E_INVAL, name
    assert mk.load_library().mk_last_error().decode() != ""


@pytest.mark.parametrize("k,no", [(48, 1024), (96, 1024), (512, 1020)])
def test_unsupported_shapes(k, no):
    a, w, f, c = good(k=k, no=no)
    assert call(a, 4, 1, w, f, c) == mk.MK_E_UNSUPPORTED
    assert mk.load_library().mk_last_error().decode() != ""


def test_bad_options():
    a, w, f, c = good()
    assert call(a, 4, 1, w, f, c, mk.ag_default_opts(grid_wgs=-1)) == mk.MK_E_INVAL
    assert call(a, 4, 1, w, f, c, mk.ag_default_opts(split_mode=9)) == mk.MK_E_INVAL
    for ph in (-1, 3):
        assert call(a, 4, 1, w, f, c, mk.ag_default_opts(phase=ph)) == mk.MK_E_INVAL
        assert b"phase" in mk.load_library().mk_last_error()
    # disable_staging (error-path testing) is 0, or 1 on the fused call only.
    for kw in (dict(disable_staging=2), dict(disable_staging=-1), dict(disable_staging=1, phase=1)):
        assert call(a, 4, 1, w, f, c, mk.ag_default_opts(**kw)) == mk.MK_E_INVAL
        assert b"disable_staging" in mk.load_library().mk_last_error()


def test_empty_shards_are_a_noop():
    assert call(desc([4, 0, 512], ptr=None), 4, 1, desc([1024, 512], ptr=FAKE), desc([0, 512], ptr=None),
                desc([0, 1024], ptr=None)) == mk.MK_OK


def test_default_opts():
    o = mk.ag_default_opts()
    assert o.split_mode == mk.MK_SPLIT_ADAPTIVE and o.grid_wgs == 0 and o.spin_timeout_us == 0
    assert o.disable_staging == 0
