"""MI355X-native per-rank ring-attention forward (mKernel's Ring Attention, one rank)
and one rank's AllGather+GEMM on the same persistent-kernel runtime.

The computation lives in the HIP library libmkra.so (C ABI in include/mkra.h and
include/mkag.h); this package is its Python binding. Build the library with
``python -m overlap_attention_amd.build``.
"""

from ._binding import (  # noqa: F401
    ag_default_opts,
    allgather_gemm,
    mk_ag_gemm_status,
    mk_allgather_gemm,
    mk_allgather_gemm_ex,
    LIB_PATH,
    MK_BF16,
    MK_E_HIP,
    MK_E_INVAL,
    MK_E_TIMEOUT,
    MK_E_UNSUPPORTED,
    MK_F32,
    MK_OK,
    MK_SPLIT_ADAPTIVE,
    MK_SPLIT_ADAPTIVE_PAPER,
    MK_SPLIT_FIXED,
    MkError,
    default_opts,
    load_library,
    mk_abi_version,
    mk_release_workspace,
    mk_ring_attn_fwd,
    mk_ring_attn_fwd_ex,
    mk_ring_attn_fwd_noalloc,
    mk_ring_attn_fwd_unfused,
    mk_ring_attn_status,
    mk_ring_attn_trace,
    ring_attn_fwd,
    tensor_desc,
)
