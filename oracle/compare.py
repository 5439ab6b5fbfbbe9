"""Parity rules between the HIP path and the oracle. TEST INFRASTRUCTURE ONLY.

* scores: |I_gpu - I_oracle| <= 1e-3 * max(|I_oracle|, 1e-3 * max_s |I_oracle(t, s)|)
  (1e-3 relative, with a row floor for scores at or near 0, where ReLU makes exact zeros
  common);
* top-k (rule T, per row): lens = min(topk, n); the first lens entries are distinct
  positions in [0, n) and every later entry is -1; if n <= topk the set is all of [0, n);
  otherwise every position in the symmetric difference of the GPU and oracle sets has an
  oracle score within 1e-5 * |s_k| of the oracle's k-th score s_k;
* attention: max |out_gpu - out_oracle| <= 2e-2 (bf16 cache) or 5e-2 (fp8 cache); lse within
  1e-3 absolute, -inf exactly for empty rows.
"""
from __future__ import annotations

import numpy as np

from .dsa_oracle import order_key

SCORE_RTOL = 1e-3
TIE_RTOL = 1e-5
OUT_TOL = {"bf16": 2e-2, "fp8_uniform": 5e-2, "fp8_uniform_fnuz": 5e-2, "fp8_ds_mla": 5e-2}
LSE_TOL = 1e-3


def scores_ok(gpu: np.ndarray, ref: np.ndarray) -> tuple[bool, str]:
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    if gpu.shape != ref.shape:
        return False, f"shape {gpu.shape} != {ref.shape}"
    if ref.size == 0:
        return gpu.size == 0, "empty"
    floor = 1e-3 * np.abs(ref).max()
    tol = SCORE_RTOL * np.maximum(np.abs(ref), floor)
    err = np.abs(gpu - ref)
    bad = np.flatnonzero(~(err <= tol))
    if bad.size:
        i = bad[0]
        return False, f"{bad.size} scores off, first at {i}: gpu {gpu[i]!r} oracle {ref[i]!r}"
    return True, f"max rel err {float((err / np.maximum(np.abs(ref), floor + 1e-300)).max()):.2e}"


def topk_ok(ref_scores: np.ndarray, k: int, gpu_idx: np.ndarray, gpu_len: int) -> tuple[bool, str]:
    n = int(ref_scores.shape[0])
    m = min(k, n)
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    if gpu_idx.ndim != 1 or gpu_idx.shape[0] < k:
        return False, f"index row of shape {gpu_idx.shape} for topk {k}"
    if int(gpu_len) != m:
        return False, f"lens {gpu_len} != {m}"
    sel = gpu_idx[:m]
    if np.any(gpu_idx[m:k] != -1):
        return False, "entries after lens are not -1"
    if np.any(sel < 0) or np.any(sel >= n):
        return False, "selected position out of range"
    if np.unique(sel).size != m:
        return False, "duplicate positions"
    if n <= k:
        return (True, "all") if set(sel.tolist()) == set(range(n)) else (False, "not all positions")
    order = order_key(ref_scores)
    ref_set = set(order[:k].tolist())
    diff = ref_set.symmetric_difference(sel.tolist())
    s_k = float(ref_scores[order[k - 1]])
    for c in diff:
        if abs(float(ref_scores[c]) - s_k) > TIE_RTOL * abs(s_k):
            return False, (f"position {c} (oracle score {ref_scores[c]!r}) differs from the oracle set "
                           f"outside the tie window around s_k={s_k!r}")
    return True, f"{len(diff)} swaps inside the tie window"


def attention_ok(out_gpu, lse_gpu, out_ref, lse_ref, fmt: str) -> tuple[bool, str]:
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    out_ref = np.asarray(out_ref, dtype=np.float64)
    if out_gpu.shape != out_ref.shape:
        return False, f"out shape {out_gpu.shape} != {out_ref.shape}"
    err = float(np.abs(out_gpu - out_ref).max()) if out_ref.size else 0.0
    if not np.isfinite(out_gpu).all():
        return False, "non-finite output"
    msg = f"out max|err| {err:.3e}"
    if err > OUT_TOL[fmt]:
        return False, msg
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        if lse_gpu.shape != lse_ref.shape:
            return False, msg + f"; lse shape {lse_gpu.shape} != {lse_ref.shape}"
        if np.isnan(lse_gpu).any():
            return False, msg + "; NaN lse"
        inf_ref = np.isneginf(lse_ref)
        if not np.array_equal(np.isneginf(lse_gpu), inf_ref):
            return False, msg + "; -inf lse mismatch"
        lerr = float(np.abs(lse_gpu[~inf_ref] - lse_ref[~inf_ref]).max()) if (~inf_ref).any() else 0.0
        msg += f", lse max|err| {lerr:.3e}"
        if lerr > LSE_TOL:
            return False, msg
    return True, msg
