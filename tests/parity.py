"""Comparison of the HIP path's results with the fp64 oracle (tolerances in one place).

Bar (stated for the method's outputs): max |out_gpu - out_ref| <= 1e-2 on the bf16
output, and 1e-3 relative error on the log-sum-exp. Two relaxations of the plain
reading of that bar are applied, and the strict figures are reported beside them:
- where |out_ref| >= 4 a correctly rounded bf16 value may already sit 1/64 away from
  the exact value, so for those elements the bar is 1e-2 + half a bf16 ulp of
  out_ref (counted in n_big_ref; out_strict_over counts elements above plain 1e-2);
- the LSE error is taken relative to max(|lse_ref|, 1), so an LSE near zero is held
  to 1e-3 absolute instead of an unbounded relative bar (lse_max_rel_err_strict is
  the plain |dlse| / |lse_ref|).
Any NaN or Inf fails.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

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
    # The bars without either relaxation, reported beside the verdict: plain 1e-2 on
    # every output element, and |dlse| / |lse_ref| (no floor at 1).
    rep["out_strict_over"] = int((err > OUT_ATOL).sum())
    with np.errstate(divide="ignore", invalid="ignore"):
        lstrict = np.abs(lse_gpu - lse_ref) / np.abs(lse_ref)
    rep["lse_max_rel_err_strict"] = float(np.nanmax(lstrict)) if lstrict.size else 0.0
    rep["ok"] = rep["finite"] and rep["out_ok"] and rep["lse_ok"]
    return rep


def compare_gemm(c_gpu, c_ref, abs_sum, k):
    """GEMM outputs (bf16, fp32 accumulation over K) against the fp64 product.

    Per element the bar is the standard bound of an fp32 accumulation, gamma_n * sum_k
    |a_k w_k| with gamma_n = n * 2^-24 and n = K/16 + 16 (K/16 accumulating MFMA steps,
    each summing 16 products), plus the final rounding to bf16: half an ulp of the
    accumulated value, whose magnitude is at most |exact| + that bound (so a sum that
    crosses into the next binade is held to that binade's ulp). abs_sum is
    sum_k |a_k w_k| per element. Returns a report dict; report['ok'] is the verdict,
    'worst_over_bar' the largest error / bar ratio."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c_gpu - c_ref)
    n = k / 16 + 16
    acc = n * 2.0 ** -24 * abs_sum
    mag = np.abs(c_ref) + acc
    bar = np.where(mag != 0, bf16_half_ulp(mag), 0.0) + acc
    rep = {"finite": bool(np.isfinite(c_gpu).all()), "max_abs_err": float(err.max()) if err.size else 0.0,
           "worst_over_bar": float((err / np.maximum(bar, 1e-300)).max()) if err.size else 0.0}
    rep["ok"] = rep["finite"] and bool((err <= bar).all())
    return rep


def oracle_rows(oracle_mod, q64, kv64, rank, causal, gqa_ratio, rows=None, workers=None, progress=False):
    """The oracle's definition evaluated one KV head at a time, the heads spread over
    threads (query heads of different KV heads never interact, so each KV head with its
    G query heads is a complete problem of its own). Each call of the oracle then sees a
    single KV head, whose key rows are contiguous. Returns (out [rows, Hq, D], lse
    [Hq, rows]) as one call over all heads would."""
    from threadpoolctl import threadpool_limits

    lq, hq, d = q64.shape
    hkv = kv64.shape[3]
    g = gqa_ratio
    if rows is None:
        rows = np.arange(lq)
    rows = np.asarray(rows, dtype=np.int64)
    if workers is None:
        workers = max(1, min(len(os.sched_getaffinity(0)), 16, hkv))

    def one(h):
        qs = np.ascontiguousarray(q64[:, h * g:(h + 1) * g])
        ks = np.ascontiguousarray(kv64[:, :, :, h:h + 1])
        return oracle_mod.ring_attention_rows(qs, ks, rank, causal, g, rows)

    out = np.empty((len(rows), hq, d))
    lse = np.empty((hq, len(rows)))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for h, (o, l) in enumerate(ex.map(one, range(hkv))):
            out[:, h * g:(h + 1) * g] = o
            lse[h * g:(h + 1) * g] = l
            if progress:
                print(f"    oracle: KV head {h + 1} of {hkv} done", flush=True)
    return out, lse


def wave_slice_rows(lq, per_slice_random=1, seed=0):
    """First and last row of every 32-row query slice, plus random rows inside each:
    every wave of every compute unit (units hold whole 32-row slices) is compared."""
    rng = np.random.default_rng(seed)
    rows = set()
    for r0 in range(0, lq, 32):
        r1 = min(lq, r0 + 32)
        rows.update((r0, r1 - 1))
        rows.update(rng.integers(r0, r1, size=per_slice_random).tolist())
    return sorted(rows)


def sample_rows(lq, n_random=24, seed=0):
    """Query rows for sampled checks: tile and wave edges, the ragged end, random rows."""
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, lq // 2, lq - 65, lq - 64, lq - 33, lq - 32, lq - 2, lq - 1}
    rng = np.random.default_rng(seed)
    rnd = set(rng.integers(0, lq, size=n_random).tolist()) if lq > 0 else set()
    return sorted(r for r in fixed | rnd if 0 <= r < lq)


def fmt(rep):
    return ", ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in rep.items())


__all__ = ["compare", "compare_gemm", "sample_rows", "wave_slice_rows", "oracle_rows", "fmt", "OUT_ATOL", "LSE_RTOL",
           "bf16_half_ulp", "math"]
