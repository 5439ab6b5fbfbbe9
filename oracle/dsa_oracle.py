"""fp64 CPU oracle of the DeepSeek Sparse Attention layer hot path.

TEST INFRASTRUCTURE ONLY. Imported by tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py; never by the HIP library or its Python binding, and it shares no code with
them. Every value is computed in float64 straight from the stored bytes (bf16 bit patterns
widened exactly, fp8 bytes through an exact decode table, UE8M0 exponents as exact powers of
two, fp32 scales as stored), with no blocking, fusion or reordering beyond the definitions.

What it computes, per query row t of request b that sees candidates s in [0, n_t):

1. Lightning-indexer score (the scoring stage of tokenspeed PR 627 "Add gluon kernel for
   DSA"; the pages name the stage but never print its formula, so this is the DeepSeek
   lightning indexer read plainly):
       I(t, s) = index_scale * sum_j w[t, j] * max(0, q_idx[t, j, :] . k[slot(b, s), :])
   with k = the bf16 key, or fp8 byte value * fp32 per-token scale for fp8 keys.
2. Top-k (the (indices, lens) pair returned by the decode top-k wrapper in the review of the
   same PR): the min(topk, n_t) candidates with the largest I, ties broken by smaller
   position, padded with -1 to topk; lens = the number selected.
3. Sparse absorbed-MLA attention (selected-attention stage of PR 627; 512 latent + 64 RoPE
   rows of tokenspeed PR 664 "gfx950 Gluon bf16 MLA decode and prefill kernels", section
   "Kernels included"): for every head h, over the listed rows i (entries -1 contribute
   nothing, radixark/miles PR 3608, section "What", padding bullet):
       l_i = softmax_scale * q[t, h, :] . c_i,   p = softmax(l),
       out[t, h, :] = sum_i p_i * c_i[:d_v],    lse[t, h] = log(sum_i exp(l_i))  (natural log)
   An empty list gives out = 0 and lse = -inf. Two lists (main + extra, aiter PR 4382 "Paged
   Sparse Attention Gluon Kernel", section "Supported formats & dtypes", two-loop bullet) are
   one softmax over their union, each list read through its own cache.
4. DeepSeek-V4 options of step 3 (radixark/miles PR 3608, section "What", forward bullet: the
   backward takes an lse in base 2 with the sink folded in). The pages name the sink without
   defining it; the reading taken: one logit per head, in the units of l_i, that joins the
   softmax denominator and carries no value row:
       out[t, h, :] = sum_i exp(l_i) c_i[:d_v] / (exp(sink_h) + sum_i exp(l_i)),
       lse[t, h] = log(exp(sink_h) + sum_i exp(l_i))
   (an empty list: out = 0, lse = sink_h). The base-2 lse is lse / ln 2.
5. Backward of step 3 with the step-4 sink (radixark/miles PR 3608, section "What": dq, and
   dKV atomic-added through the clamped indices; the pages give no formula, so this is the
   exact gradient of the forward above, for one list). For an upstream gradient dout[h, :]:
       p_i = exp(l_i - lse_h),  p_sink = exp(sink_h - lse_h),  D_h = dout[h, :] . out[h, :],
       dl_i = p_i * (dout[h, :] . c_i[:d_v] - D_h),
       dq[h, :] = softmax_scale * sum_i dl_i * c_i[:d_qk],
       dc_i[:d_qk] += softmax_scale * dl_i * q[h, :],   dc_i[:d_v] += p_i * dout[h, :],
       dsink_h = -p_sink * D_h
   summed over heads for dc_i; an entry listed twice contributes twice (each listed entry is
   its own term of the softmax). The backward is handed the forward's outputs (the same PR's
   forward bullet: the backward takes the forward's lse); when they are given, lse_h and
   out[h, :] are taken as given (p_i and p_sink from that lse, D_h from that out), which is
   exactly the gradient above when they equal the forward's exact values.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------- stored formats


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of an fp32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _fp8_e4m3fn_table() -> np.ndarray:
    """Value of every OCP e4m3fn byte (aiter PR 4382, header: OCP = float8_e4m3fn, bias 7).

    Layout s.eeee.mmm: exponent bias 7; e = 0 is subnormal (m / 8 * 2^-6); no infinities;
    S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    t = np.empty(256, dtype=np.float64)
    for byte in range(256):
        sign = -1.0 if byte & 0x80 else 1.0
        e = (byte >> 3) & 0xF
        m = byte & 0x7
        if e == 0xF and m == 0x7:
            t[byte] = math.nan
        elif e == 0:
            t[byte] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[byte] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


FP8_E4M3FN = _fp8_e4m3fn_table()


def _fp8_e4m3fnuz_table() -> np.ndarray:
    """Value of every fnuz e4m3 byte (aiter PR 4382, section "fp8 flavors": float8_e4m3fnuz,
    exponent bias 8).

    Layout s.eeee.mmm: bias 8; e = 0 is subnormal (m / 8 * 2^-7); no infinities and no negative
    zero: byte 0x80 is the only NaN, so S.1111.111 is finite, 1.875 * 2^7 = 240.
    """
    t = np.empty(256, dtype=np.float64)
    for byte in range(256):
        sign = -1.0 if byte & 0x80 else 1.0
        e = (byte >> 3) & 0xF
        m = byte & 0x7
        if byte == 0x80:
            t[byte] = math.nan
        elif e == 0:
            t[byte] = sign * (m / 8.0) * 2.0 ** (1 - 8)
        else:
            t[byte] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)
    return t


FP8_E4M3FNUZ = _fp8_e4m3fnuz_table()


def ue8m0_to_f64(e: np.ndarray) -> np.ndarray:
    """UE8M0 exponent byte -> 2^(e - 127) (aiter PR 4382, fp8_ds_mla dequant bullet).

    Byte 255 is never produced by the cache writer; reading it is an error here.
    """
    e = np.asarray(e, dtype=np.int64)
    if np.any(e == 255):
        raise ValueError("UE8M0 byte 255 in a scale")
    return np.ldexp(1.0, e - 127)


# --------------------------------------------------------------------------- addressing


def slots_of(pool, b: int, positions: np.ndarray) -> np.ndarray:
    """Logical positions of request b -> physical token slots.

    With a page table: slot = table[b, s // page] * page + s % page (paged MLA cache, page 64,
    PR 664; block table on the decode top-k wrapper, PR 627 review). Without one the cache is
    packed and request b starts at req_base[b].
    """
    s = np.asarray(positions, dtype=np.int64)
    if pool.block_table is not None:
        P = int(pool.page_size)
        pages = np.asarray(pool.block_table[b], dtype=np.int64)[s // P]
        return pages * P + s % P
    return int(pool.req_base[b]) + s


def key_rows(kpool, b: int, positions: np.ndarray) -> np.ndarray:
    """Indexer keys of the given positions, float64 [n, di]."""
    slots = slots_of(kpool, b, positions)
    if kpool.dtype == "bf16":
        return bf16_to_f64(kpool.data[slots])
    if kpool.dtype == "fp8":
        vals = FP8_E4M3FN[kpool.data[slots]]
        return vals * kpool.scale[slots].astype(np.float64)[:, None]
    raise ValueError(kpool.dtype)


def kv_rows(pool, b: int, positions: np.ndarray) -> np.ndarray:
    """Latent rows of the given positions, dequantised to float64 [n, d_nope + d_rope].

    fp8_uniform (PR 4382, "Uniform fp8 pool - 2D"): x = fp8(byte[slot, c]) * scale[slot, c // 64];
    fp8_uniform_fnuz: the same with the fnuz decoding of the bytes (section "fp8 flavors").
    fp8_ds_mla (PR 4382, "Packed fp8 fp8_ds_mla - 3D"): slot -> page = slot // block,
    pos = slot % block; the page holds block x 576 data bytes then block x 8 scale bytes;
    NoPE byte c of the token sits at pos * 576 + c and is scaled by 2^(e_g - 127) with
    e_g = the scale byte at block * 576 + pos * 8 + c // 64; the 64 RoPE values are bf16 at
    pos * 576 + 448 + 2 i (little endian) and are not scaled.
    """
    slots = slots_of(pool, b, positions)
    if pool.fmt == "bf16":
        return bf16_to_f64(pool.data[slots])
    if pool.fmt in ("fp8_uniform", "fp8_uniform_fnuz"):
        if pool.fmt == "fp8_uniform":
            vals = FP8_E4M3FN[pool.data[slots]]
        else:
            if np.any(pool.data[slots] == 0x80):
                raise ValueError("fnuz NaN byte 0x80 in a cache row")
            vals = FP8_E4M3FNUZ[pool.data[slots]]
        groups = np.arange(vals.shape[1]) // 64
        return vals * pool.scales[slots][:, groups].astype(np.float64)
    if pool.fmt == "fp8_ds_mla":
        blk = int(pool.page_size)
        page = slots // blk
        pos = slots % blk
        n_nope, n_rope = pool.d_nope, pool.d_rope
        data_off = pos * 576
        nope_bytes = pool.data[page[:, None], data_off[:, None] + np.arange(n_nope)[None, :]]
        scale_off = blk * 576 + pos * 8
        exps = pool.data[page[:, None], scale_off[:, None] + np.arange(n_nope // 64)[None, :]]
        nope = FP8_E4M3FN[nope_bytes] * np.repeat(ue8m0_to_f64(exps), 64, axis=1)
        lo = pool.data[page[:, None], data_off[:, None] + n_nope + 2 * np.arange(n_rope)[None, :]]
        hi = pool.data[page[:, None], data_off[:, None] + n_nope + 2 * np.arange(n_rope)[None, :] + 1]
        rope = bf16_to_f64(lo.astype(np.uint16) | (hi.astype(np.uint16) << np.uint16(8)))
        return np.concatenate([nope, rope], axis=1)
    raise ValueError(pool.fmt)


# --------------------------------------------------------------------------- the three steps


def index_scores_row(prob, t: int, positions: np.ndarray | None = None) -> np.ndarray:
    """I(t, s) for s in [0, n_t) (or for the given positions only), float64."""
    b = int(prob.row_req[t])
    n = int(prob.row_len[t])
    pos = np.arange(n) if positions is None else np.asarray(positions, dtype=np.int64)
    keys = key_rows(prob.kpool, b, pos)                         # [n, di]
    q = bf16_to_f64(prob.q_idx[t])                              # [Hi, di]
    w = prob.w[t].astype(np.float64)                            # [Hi]
    dots = q @ keys.T                                           # [Hi, n]
    return float(prob.index_scale) * (w @ np.maximum(dots, 0.0))


def order_key(scores: np.ndarray) -> np.ndarray:
    """Positions sorted by (score descending, position ascending)."""
    n = scores.shape[0]
    return np.lexsort((np.arange(n), -scores))


def topk_row(scores: np.ndarray, k: int) -> tuple[np.ndarray, int]:
    """(indices int32 [k] padded with -1, lens) of the min(k, n) best positions."""
    n = scores.shape[0]
    m = min(k, n)
    idx = np.full(k, -1, dtype=np.int32)
    idx[:m] = order_key(scores)[:m]
    return idx, m


def attention_row(prob, t: int, idx_main: np.ndarray, idx_extra: np.ndarray | None = None):
    """Sparse MLA attention of row t over the listed rows. Returns (out [H, d_v], lse [H]).

    prob.sink (float32 [H] or None) and prob.lse_log2 (bool) are the DeepSeek-V4 options of
    step 4 of the module description; absent attributes mean no sink and a natural-log lse."""
    b = int(prob.row_req[t])
    parts = []
    for pool, lst in ((prob.kv, idx_main), (prob.extra_kv, idx_extra)):
        if lst is None or pool is None:
            continue
        lst = np.asarray(lst, dtype=np.int64)
        keep = lst[lst != -1]
        if keep.size:
            parts.append(kv_rows(pool, b, keep))
    H, d_v = prob.H, prob.d_v
    sink = getattr(prob, "sink", None)
    sink = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    base = math.log(2.0) if getattr(prob, "lse_log2", False) else 1.0
    if not parts:
        return np.zeros((H, d_v)), sink / base
    rows = np.concatenate(parts, axis=0)                        # [n, D]
    q = bf16_to_f64(prob.q[t])                                  # [H, d_qk]
    out, lse = attention_math(q, rows, sink, float(prob.softmax_scale), prob.d_qk, d_v)
    return out, lse / base


def attention_math(q: np.ndarray, rows: np.ndarray, sink: np.ndarray, scale: float, d_qk: int,
                   d_v: int):
    """Step 3/4 on float64 arrays: q [H, d_qk], rows [n >= 1, D], sink [H] (-inf: none).
    Returns (out [H, d_v], natural-log lse [H])."""
    logits = scale * (q @ rows[:, :d_qk].T)                     # [H, n]
    m = np.maximum(logits.max(axis=1), sink)[:, None]           # finite: there is a row
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True) + np.exp(sink[:, None] - m)
    out = (e @ rows[:, :d_v]) / z
    lse = (m + np.log(z))[:, 0]
    return out, lse


def attention_backward_math(q: np.ndarray, rows: np.ndarray, sink: np.ndarray, scale: float,
                            d_qk: int, d_v: int, dout: np.ndarray, out: np.ndarray | None = None,
                            lse: np.ndarray | None = None):
    """Step 5 on float64 arrays (q [H, d_qk], rows [n >= 1, D], sink [H], dout [H, d_v]).
    out [H, d_v] and lse [H] (natural log), when given, are the forward's outputs as handed to
    the backward; otherwise the exact forward values are used.
    Returns (dq [H, d_qk], drows [n, max(d_qk, d_v)] per listed entry, dsink [H])."""
    logits = scale * (q @ rows[:, :d_qk].T)                     # [H, n]
    if lse is None:
        m = np.maximum(logits.max(axis=1), sink)[:, None]
        lse = m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True) + np.exp(sink[:, None] - m))
    else:
        lse = np.asarray(lse, dtype=np.float64)[:, None]
    p = np.exp(logits - lse)                                    # [H, n]
    p_sink = np.exp(sink[:, None] - lse)[:, 0]                  # [H]
    if out is None:
        out = p @ rows[:, :d_v]                                 # [H, d_v]
    D = (dout * np.asarray(out, dtype=np.float64)).sum(axis=1)  # [H]
    dp = dout @ rows[:, :d_v].T                                 # [H, n]
    dl = p * (dp - D[:, None])                                  # [H, n]
    dq = scale * (dl @ rows[:, :d_qk])                          # [H, d_qk]
    drows = np.zeros((rows.shape[0], max(d_qk, d_v)))
    drows[:, :d_qk] += scale * (dl.T @ q)
    drows[:, :d_v] += p.T @ dout
    dsink = -p_sink * D
    return dq, drows, dsink


def attention_backward_row(prob, t: int, idx: np.ndarray, dout: np.ndarray,
                           out: np.ndarray | None = None, lse: np.ndarray | None = None):
    """Step 5 for row t over one list (main cache): dout float64 [H, d_v]. out [H, d_v] and
    lse [H] (in the base prob.lse_log2 names), when given, are the forward's outputs handed to
    the backward. Returns (dq [H, d_qk], slots [n] of the valid listed entries in list order,
    drows [n, D], dsink [H]); an empty list gives zeros."""
    b = int(prob.row_req[t])
    lst = np.asarray(idx, dtype=np.int64)
    keep = lst[lst != -1]
    H = prob.H
    sink = getattr(prob, "sink", None)
    sink = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    D = max(prob.d_qk, prob.d_v)
    if keep.size == 0:
        return np.zeros((H, prob.d_qk)), np.zeros(0, np.int64), np.zeros((0, D)), np.zeros(H)
    rows = kv_rows(prob.kv, b, keep)
    q = bf16_to_f64(prob.q[t])
    if lse is not None:
        base = math.log(2.0) if getattr(prob, "lse_log2", False) else 1.0
        lse = np.asarray(lse, dtype=np.float64) * base
    dq, drows, dsink = attention_backward_math(q, rows, sink, float(prob.softmax_scale), prob.d_qk,
                                               prob.d_v, np.asarray(dout, dtype=np.float64),
                                               out=out, lse=lse)
    return dq, slots_of(prob.kv, b, keep), drows, dsink


def layer_row(prob, t: int) -> dict:
    """Whole layer for row t: scores, top-k, attention over the oracle's own selection."""
    scores = index_scores_row(prob, t)
    idx, n_sel = topk_row(scores, prob.topk)
    out, lse = attention_row(prob, t, idx)
    return {"scores": scores, "idx": idx, "lens": n_sel, "out": out, "lse": lse}
