"""Comparison of the HIP path's results with the fp64 oracle (tolerances in one place).

Bar (stated for the method's outputs): max |out_gpu - out_ref| <= 1e-2 on the bf16
output, and |lse_gpu - lse_ref| / max(|lse_ref|, 1) <= 1e-3 on the log-sum-exp.
Where |out_ref| >= 4 a correctly rounded bf16 value may already sit 1/64 away from
the exact value, so for those elements the bar is 1e-2 + half a bf16 ulp of out_ref
(the only relaxation; counted and reported). Any NaN or Inf fails.
"""

import math

import numpy as np

OUT_ATOL = 1e-2
LSE_RTOL = 1e-3


def bf16_half_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, np.finfo(np.float64).tiny)))
    return 0.5 * np.exp2(e - 7)  # bf16 keeps 8 significant bits


def compare(out_gpu, lse_gpu, out_ref, lse_ref):
    """Returns a report dict; report['ok'] is the verdict."""
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    rep = {}
    rep["finite"] = bool(np.isfinite(out_gpu).all() and np.isfinite(lse_gpu).all())
    err = np.abs(out_gpu - out_ref)
    big = np.abs(out_ref) >= 4.0
    bar = np.where(big, OUT_ATOL + bf16_half_ulp(out_ref), OUT_ATOL)
    rep["max_abs_err"] = float(err.max()) if err.size else 0.0
    rep["n_big_ref"] = int(big.sum())
    rep["out_ok"] = bool((err <= bar).all())
    lerr = np.abs(lse_gpu - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    rep["lse_max_rel_err"] = float(lerr.max()) if lerr.size else 0.0
    rep["lse_ok"] = bool((lerr <= LSE_RTOL).all())
    rep["ok"] = rep["finite"] and rep["out_ok"] and rep["lse_ok"]
    return rep


def sample_rows(lq, n_random=24, seed=0):
    """Query rows for sampled checks: tile and wave edges, the ragged end, random rows."""
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, lq // 2, lq - 65, lq - 64, lq - 33, lq - 32, lq - 2, lq - 1}
    rng = np.random.default_rng(seed)
    rnd = set(rng.integers(0, lq, size=n_random).tolist()) if lq > 0 else set()
    return sorted(r for r in fixed | rnd if 0 <= r < lq)


def fmt(rep):
    return ", ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in rep.items())


__all__ = ["compare", "sample_rows", "fmt", "OUT_ATOL", "LSE_RTOL", "bf16_half_ulp", "math"]
