"""ctypes binding of libmkra.so (include/mkra.h). Argument marshalling only.

The functions keep the C names. PyTorch supplies device memory and the stream; every
step of the computation runs in the library's HIP kernel. If the library is missing
this module raises on import of the entry points: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmkra.so")

MK_OK, MK_E_INVAL, MK_E_UNSUPPORTED, MK_E_HIP, MK_E_TIMEOUT = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "MK_OK", 1: "MK_E_INVAL", 2: "MK_E_UNSUPPORTED", 3: "MK_E_HIP", 4: "MK_E_TIMEOUT"}
MK_BF16, MK_F32 = 1, 2
MK_SPLIT_ADAPTIVE, MK_SPLIT_FIXED, MK_SPLIT_ADAPTIVE_PAPER = 0, 1, 2


class mk_tensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 5),
        ("stride", ctypes.c_int64 * 5),
    ]


class mk_ring_attn_opts(ctypes.Structure):
    _fields_ = [
        ("split_mode", ctypes.c_int32),
        ("fixed_staging_wgs", ctypes.c_int32),
        ("initial_staging_wgs", ctypes.c_int32),
        ("grid_wgs", ctypes.c_int32),
        ("spin_timeout_us", ctypes.c_int64),
        ("controller_period_us", ctypes.c_int32),
        ("trace", ctypes.c_int32),
        ("trace_capacity", ctypes.c_int32),
        ("disable_staging", ctypes.c_int32),
        ("stage_delay_ticks", ctypes.c_int32),
        ("debug_flags", ctypes.c_int32),
        ("steps_per_task", ctypes.c_int32),
        ("tail_steps", ctypes.c_int32),
        ("tail_steps_per_task", ctypes.c_int32),
        ("parallel_steps", ctypes.c_int32),
        ("stage_pieces", ctypes.c_int32),
    ]


class mk_ring_attn_stats(ctypes.Structure):
    _fields_ = [
        ("status", ctypes.c_int32),
        ("grid_wgs", ctypes.c_int32),
        ("n_units", ctypes.c_int32),
        ("n_steps", ctypes.c_int32),
        ("n_stage_tiles", ctypes.c_int32),
        ("n_stage_tasks", ctypes.c_int32),
        ("compute_tasks_done", ctypes.c_int32),
        ("staging_tasks_done", ctypes.c_int32),
        ("assist_tasks", ctypes.c_int32),
        ("initial_target", ctypes.c_int32),
        ("final_target", ctypes.c_int32),
        ("max_staging_wgs", ctypes.c_int32),
        ("controller_updates", ctypes.c_int32),
        ("role_switches", ctypes.c_int32),
        ("compute_busy_ticks", ctypes.c_int64),
        ("compute_wait_ticks", ctypes.c_int64),
        ("staging_busy_ticks", ctypes.c_int64),
        ("staging_wait_ticks", ctypes.c_int64),
        ("kernel_ticks", ctypes.c_int64),
        ("trace_records", ctypes.c_int64),
        ("debug_mismatches", ctypes.c_int64),
        ("wg_cycles", ctypes.c_int64),
        ("wg_ticks", ctypes.c_int64),
        ("steps_per_task", ctypes.c_int32),
        ("step_groups", ctypes.c_int32),
        ("parallel_steps", ctypes.c_int32),
        ("stage_pieces", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_ if not name.startswith("reserved")}


class mk_ag_gemm_opts(ctypes.Structure):
    _fields_ = [
        ("split_mode", ctypes.c_int32),
        ("fixed_staging_wgs", ctypes.c_int32),
        ("initial_staging_wgs", ctypes.c_int32),
        ("grid_wgs", ctypes.c_int32),
        ("spin_timeout_us", ctypes.c_int64),
        ("controller_period_us", ctypes.c_int32),
        ("phase", ctypes.c_int32),
        ("disable_staging", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 3),
    ]


class mk_ag_gemm_stats(ctypes.Structure):
    _fields_ = [
        ("status", ctypes.c_int32),
        ("grid_wgs", ctypes.c_int32),
        ("compute_tiles", ctypes.c_int32),
        ("staging_tasks", ctypes.c_int32),
        ("compute_done", ctypes.c_int32),
        ("staging_done", ctypes.c_int32),
        ("assist_tasks", ctypes.c_int32),
        ("controller_updates", ctypes.c_int32),
        ("max_staging_wgs", ctypes.c_int32),
        ("final_target", ctypes.c_int32),
        ("compute_busy_ticks", ctypes.c_int64),
        ("compute_wait_ticks", ctypes.c_int64),
        ("staging_busy_ticks", ctypes.c_int64),
        ("kernel_ticks", ctypes.c_int64),
        ("wg_cycles", ctypes.c_int64),
        ("wg_ticks", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class mk_trace_record(ctypes.Structure):
    _fields_ = [("t", ctypes.c_uint64), ("wg", ctypes.c_int32), ("kind", ctypes.c_int32), ("v", ctypes.c_int64 * 6)]


# Every function the header declares, with its ctypes signature.
_PROTOTYPES = {
    "mk_ring_attn_fwd": (ctypes.c_int, [ctypes.POINTER(mk_tensor), ctypes.POINTER(mk_tensor), ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(mk_tensor),
                                        ctypes.POINTER(mk_tensor), ctypes.c_void_p]),
    "mk_ring_attn_fwd_ex": (ctypes.c_int, [ctypes.POINTER(mk_tensor), ctypes.POINTER(mk_tensor), ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(mk_tensor),
                                           ctypes.POINTER(mk_tensor), ctypes.c_void_p,
                                           ctypes.POINTER(mk_ring_attn_opts), ctypes.POINTER(mk_ring_attn_stats)]),
    "mk_ring_attn_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(mk_tensor), ctypes.POINTER(mk_tensor), ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(mk_tensor),
                                                ctypes.POINTER(mk_tensor), ctypes.c_void_p]),
    "mk_ring_attn_fwd_unfused": (ctypes.c_int, [ctypes.POINTER(mk_tensor), ctypes.POINTER(mk_tensor), ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(mk_tensor),
                                                ctypes.POINTER(mk_tensor), ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_int]),
    "mk_ring_attn_default_opts": (None, [ctypes.POINTER(mk_ring_attn_opts)]),
    "mk_ring_attn_status": (ctypes.c_int, [ctypes.c_void_p]),
    "mk_ring_attn_trace": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(mk_trace_record), ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]),
    "mk_allgather_gemm": (ctypes.c_int, [ctypes.POINTER(mk_tensor), ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(mk_tensor), ctypes.POINTER(mk_tensor),
                                         ctypes.POINTER(mk_tensor), ctypes.c_void_p]),
    "mk_allgather_gemm_ex": (ctypes.c_int, [ctypes.POINTER(mk_tensor), ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(mk_tensor), ctypes.POINTER(mk_tensor),
                                            ctypes.POINTER(mk_tensor), ctypes.c_void_p,
                                            ctypes.POINTER(mk_ag_gemm_opts), ctypes.POINTER(mk_ag_gemm_stats)]),
    "mk_ag_gemm_default_opts": (None, [ctypes.POINTER(mk_ag_gemm_opts)]),
    "mk_ag_gemm_status": (ctypes.c_int, [ctypes.c_void_p]),
    "mk_last_error": (ctypes.c_char_p, []),
    "mk_release_workspace": (None, []),
    "mk_abi_version": (ctypes.c_int, []),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmkra.so (built in-tree by overlap_attention_amd.build). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m overlap_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(status: int):
    if status != MK_OK:
        raise MkError(status, load_library().mk_last_error().decode())


def tensor_desc(t, dtype_code: Optional[int] = None) -> mk_tensor:
    """Descriptor of a torch tensor (pointer, dtype, shape, strides in elements)."""
    import torch

    if dtype_code is None:
        dtype_code = {torch.bfloat16: MK_BF16, torch.float32: MK_F32}.get(t.dtype, 0)
    d = mk_tensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = dtype_code
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def default_opts(**overrides) -> mk_ring_attn_opts:
    o = mk_ring_attn_opts()
    load_library().mk_ring_attn_default_opts(ctypes.byref(o))
    for k, v in overrides.items():
        if not hasattr(o, k):
            raise KeyError(k)
        setattr(o, k, v)
    return o


def _stream_ptr(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def mk_ring_attn_fwd(q, kv_chunks, n_chunks: int, rank: int, causal: bool, gqa_ratio: int, out, lse,
                     stream=None) -> None:
    """Thin call of mk_ring_attn_fwd on torch tensors (all on the current GPU)."""
    lib = load_library()
    qd, kd, od, ld = tensor_desc(q), tensor_desc(kv_chunks), tensor_desc(out), tensor_desc(lse)
    _check(lib.mk_ring_attn_fwd(ctypes.byref(qd), ctypes.byref(kd), n_chunks, rank, int(bool(causal)), gqa_ratio,
                                ctypes.byref(od), ctypes.byref(ld), _stream_ptr(stream)))


def mk_ring_attn_fwd_ex(q, kv_chunks, n_chunks: int, rank: int, causal: bool, gqa_ratio: int, out, lse,
                        stream=None, opts: Optional[mk_ring_attn_opts] = None, want_stats: bool = False):
    """Thin call of mk_ring_attn_fwd_ex; returns the stats dict when want_stats."""
    lib = load_library()
    qd, kd, od, ld = tensor_desc(q), tensor_desc(kv_chunks), tensor_desc(out), tensor_desc(lse)
    st = mk_ring_attn_stats() if want_stats else None
    _check(lib.mk_ring_attn_fwd_ex(ctypes.byref(qd), ctypes.byref(kd), n_chunks, rank, int(bool(causal)), gqa_ratio,
                                   ctypes.byref(od), ctypes.byref(ld), _stream_ptr(stream),
                                   ctypes.byref(opts) if opts is not None else None,
                                   ctypes.byref(st) if st is not None else None))
    return st.as_dict() if st is not None else None


def mk_ring_attn_fwd_noalloc(q, kv_chunks, n_chunks: int, rank: int, causal: bool, gqa_ratio: int, out, lse,
                             stream=None) -> None:
    """Thin call of mk_ring_attn_fwd_noalloc (the entry point that allocates no device
    memory) on torch tensors the caller allocated."""
    lib = load_library()
    qd, kd, od, ld = tensor_desc(q), tensor_desc(kv_chunks), tensor_desc(out), tensor_desc(lse)
    _check(lib.mk_ring_attn_fwd_noalloc(ctypes.byref(qd), ctypes.byref(kd), n_chunks, rank, int(bool(causal)),
                                        gqa_ratio, ctypes.byref(od), ctypes.byref(ld), _stream_ptr(stream)))


def mk_ring_attn_fwd_unfused(q, kv_chunks, n_chunks: int, rank: int, causal: bool, gqa_ratio: int, out, lse,
                             copy_stream, copy_wgs: int, stream=None) -> None:
    """Thin call of mk_ring_attn_fwd_unfused (the two-stream unfused baseline); copy_stream
    is a torch stream other than `stream`."""
    lib = load_library()
    qd, kd, od, ld = tensor_desc(q), tensor_desc(kv_chunks), tensor_desc(out), tensor_desc(lse)
    _check(lib.mk_ring_attn_fwd_unfused(ctypes.byref(qd), ctypes.byref(kd), n_chunks, rank, int(bool(causal)),
                                        gqa_ratio, ctypes.byref(od), ctypes.byref(ld), _stream_ptr(stream),
                                        _stream_ptr(copy_stream), copy_wgs))


def mk_ring_attn_status(stream=None) -> int:
    """Status of earlier calls on the stream; raises MkError unless MK_OK."""
    _check(load_library().mk_ring_attn_status(_stream_ptr(stream)))
    return MK_OK


def mk_ring_attn_trace(stream=None, capacity: int = 1 << 20):
    """Trace records of the last traced call on the stream, as a list of tuples
    (t, wg, kind, v0..v5)."""
    lib = load_library()
    buf = (mk_trace_record * capacity)()
    n = ctypes.c_int64(0)
    _check(lib.mk_ring_attn_trace(_stream_ptr(stream), buf, capacity, ctypes.byref(n)))
    return [(r.t, r.wg, r.kind) + tuple(r.v) for r in buf[:n.value]]


def mk_release_workspace() -> None:
    load_library().mk_release_workspace()


def mk_abi_version() -> int:
    return load_library().mk_abi_version()


def ring_attn_fwd(q, kv_chunks, rank: int, causal: bool, gqa_ratio: int, opts: Optional[mk_ring_attn_opts] = None,
                  want_stats: bool = False, stream=None) -> Tuple:
    """Allocates out [Lq, Hq, D] bf16 and lse [Hq, Lq] fp32 and runs the forward.

    Returns (out, lse) or (out, lse, stats) when want_stats.
    """
    import torch

    lq, hq, _ = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((hq, lq), dtype=torch.float32, device=q.device)
    stats = mk_ring_attn_fwd_ex(q, kv_chunks, kv_chunks.shape[0], rank, causal, gqa_ratio, out, lse, stream=stream,
                                opts=opts, want_stats=want_stats)
    return (out, lse, stats) if want_stats else (out, lse)


# ------------------------------------------------------------------ AllGather+GEMM

def ag_default_opts(**overrides) -> mk_ag_gemm_opts:
    o = mk_ag_gemm_opts()
    load_library().mk_ag_gemm_default_opts(ctypes.byref(o))
    for k, v in overrides.items():
        if not hasattr(o, k):
            raise KeyError(k)
        setattr(o, k, v)
    return o


def mk_allgather_gemm(a_shards, n_ranks: int, rank: int, w, a_full, c, stream=None) -> None:
    """Thin call of mk_allgather_gemm on torch tensors (all on the current GPU)."""
    lib = load_library()
    ad, wd, fd, cd = tensor_desc(a_shards), tensor_desc(w), tensor_desc(a_full), tensor_desc(c)
    _check(lib.mk_allgather_gemm(ctypes.byref(ad), n_ranks, rank, ctypes.byref(wd), ctypes.byref(fd),
                                 ctypes.byref(cd), _stream_ptr(stream)))


def mk_allgather_gemm_ex(a_shards, n_ranks: int, rank: int, w, a_full, c, stream=None,
                         opts: Optional[mk_ag_gemm_opts] = None, want_stats: bool = False):
    """Thin call of mk_allgather_gemm_ex; returns the stats dict when want_stats."""
    lib = load_library()
    ad, wd, fd, cd = tensor_desc(a_shards), tensor_desc(w), tensor_desc(a_full), tensor_desc(c)
    st = mk_ag_gemm_stats() if want_stats else None
    _check(lib.mk_allgather_gemm_ex(ctypes.byref(ad), n_ranks, rank, ctypes.byref(wd), ctypes.byref(fd),
                                    ctypes.byref(cd), _stream_ptr(stream),
                                    ctypes.byref(opts) if opts is not None else None,
                                    ctypes.byref(st) if st is not None else None))
    return st.as_dict() if st is not None else None


def mk_ag_gemm_status(stream=None) -> int:
    """Status of earlier AllGather+GEMM calls on the stream; raises MkError unless MK_OK."""
    _check(load_library().mk_ag_gemm_status(_stream_ptr(stream)))
    return MK_OK


def allgather_gemm(a_shards, rank: int, w, opts: Optional[mk_ag_gemm_opts] = None, want_stats: bool = False,
                   stream=None) -> Tuple:
    """Allocates a_full [N*M_loc, K] and c [N*M_loc, N_out] (bf16) and runs one rank's
    AllGather+GEMM. Returns (a_full, c) or (a_full, c, stats) when want_stats."""
    import torch

    n, m_loc, k = a_shards.shape
    a_full = torch.empty((n * m_loc, k), dtype=a_shards.dtype, device=a_shards.device)
    c = torch.empty((n * m_loc, w.shape[0]), dtype=a_shards.dtype, device=a_shards.device)
    stats = mk_allgather_gemm_ex(a_shards, n, rank, w, a_full, c, stream=stream, opts=opts, want_stats=want_stats)
    return (a_full, c, stats) if want_stats else (a_full, c)
