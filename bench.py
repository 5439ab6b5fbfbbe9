#!/usr/bin/env python3
"""DSA layer benchmark on one MI355X: scores + top-k + sparse MLA attention at 128k decode.

One step = one fused dsa_decode call (indexer scores over every cached token, top-k, sparse
MLA attention over the selected latent rows) for one batch of seeded synthetic inputs already
resident in HBM. The headline is the cold per-layer time: before every step a 1 GiB read
evicts L2 and the 256 MiB last-level cache (outside the timed events), as between layers of
a real model whose caches far exceed them. The warm time (steps back to back) is reported
beside it.

Prints one JSON line (last line of stdout).
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

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth
# the pages' figure for this metric and shape (context only: another GPU generation's kernel)
PAGE_128K_DECODE_US = 411.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def keys_read(prob):
    """Index keys the method must read: rows of one request share its keys, so each request
    counts its longest row once."""
    import numpy as np
    req = np.asarray(prob.row_req)
    lens = np.asarray(prob.row_len)
    return int(sum(int(lens[req == b].max()) for b in np.unique(req)))


def algorithmic_bytes(prob):
    """What the method must move per layer (decode, one row per request)."""
    T, H, topk = prob.T, prob.H, prob.topk
    n = keys_read(prob)
    key_b = 2 if prob.kpool.dtype == "bf16" else 1
    keys = n * prob.di * key_b + (n * 4 if prob.kpool.dtype == "fp8" else 0)
    row_b = {"bf16": 2 * prob.d_qk, "fp8_uniform": prob.d_qk + 4 * prob.d_qk // 64, "fp8_ds_mla": 584}[prob.kv.fmt]
    gathered = T * min(topk, int(prob.row_len.max())) * row_b
    qio = T * (H * prob.d_qk * 2 + prob.Hi * prob.di * 2 + prob.Hi * 4 + H * prob.d_v * 2 + H * 4 + topk * 4)
    return {"keys": keys, "gathered_rows": gathered, "q_out_idx": qio, "total": keys + gathered + qio}


def kernel_bytes(prob, kernel):
    """Algorithmic bytes one launch of `kernel` must move (decode, one row per request):
    what the step reads and writes by definition, not what the implementation adds."""
    T, n = prob.T, keys_read(prob)
    topk = prob.topk
    if kernel.startswith("index_scores"):
        # every key (and fp8 scale) read once, every score written once, the query heads,
        # weights and page-table entries read once
        key_b = 2 if prob.kpool.dtype == "bf16" else 1
        per_cand = prob.di * key_b + 4 + (4 if prob.kpool.dtype == "fp8" else 0)
        pages = (n + prob.kpool.page_size - 1) // prob.kpool.page_size
        return n * per_cand + T * (prob.Hi * prob.di * 2 + prob.Hi * 4) + pages * 4
    if kernel.startswith("topk"):
        # the scores read once, the index list written once
        return n * 4 + T * topk * 4
    if kernel == "sparse_mla":
        row_b = {"bf16": 2 * prob.d_qk, "fp8_uniform": prob.d_qk + 4 * prob.d_qk // 64,
                 "fp8_ds_mla": 584}[prob.kv.fmt]
        rows = sum(min(topk, int(x)) for x in prob.row_len)
        return rows * row_b + rows * 4 + T * prob.H * prob.d_qk * 2
    return None


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "deepseek_sparse_attention_indexer_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def prefill_indexer(dsa, to_device, workloads, torch, dev, reps=5):
    """The indexer's score kernel on the causal prefill (segments 8192 + 1, 64 x 128 indexer
    heads): MFMA-equivalent rate over the dense bf16 peak."""
    import numpy as np
    prob = workloads.causal_prefill((8192, 1), make_attn=False, name="causal_prefill_8k")
    d = to_device(prob, dev)
    ld = ((prob.n_max + 63) // 64) * 64
    logits = torch.empty(prob.T, ld, dtype=torch.float32, device=dev)
    pairs = int(prob.row_len.astype(np.int64).sum())
    flops = pairs * 2 * prob.Hi * prob.di

    def run():
        dsa.dsa_index_scores(d.q_idx, d.w, d.keys, d.rows, prob.Hi, prob.di, prob.index_scale, logits)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    dsa.dsa_profile_enable(True)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    prof = dsa.dsa_profile_collect()
    dsa.dsa_profile_enable(False)
    name, rec = max(prof.items(), key=lambda kv: kv[1]["total_ms"])
    us = rec["total_ms"] / rec["count"] * 1e3
    achieved = flops / (us * 1e-6) / 1e12
    # the same launches with the GPU idle for 20 ms before each: sustained back-to-back matrix
    # work lowers the clock, so both figures are given (frac is the back-to-back one)
    dsa.dsa_profile_enable(True)
    for _ in range(reps):
        torch.cuda.synchronize()
        time.sleep(0.02)
        run()
    torch.cuda.synchronize()
    prof_i = dsa.dsa_profile_collect()
    dsa.dsa_profile_enable(False)
    us_i = prof_i[name]["total_ms"] / prof_i[name]["count"] * 1e3
    achieved_i = flops / (us_i * 1e-6) / 1e12
    return {"workload": "causal_prefill_8k", "kernel": name, "rows": int(prob.T), "score_pairs": pairs,
            "gflop": round(flops / 1e9, 2), "avg_us": round(us, 1), "bound": "mfma",
            "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "isolated_us": round(us_i, 1), "isolated_frac": round(achieved_i / MFMA_BF16_PEAK_TFLOPS, 4),
            "timing": "HIP events from each dispatch, inputs resident (8193 rows x 64 x 128 bf16); "
                      "avg_us back to back, isolated_us after 20 ms of idle GPU"}


def calibration(torch, dev, reps=5):
    """Measured ceilings beside the published ones: a plain device copy (HBM read + write) and a
    dense bf16 GEMM from the vendor library (torch.mm on contiguous 8192^3 operands)."""
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)       # 512 MiB
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = None
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best * 1e-3

    t_copy = timed(lambda: dst.copy_(src))
    t_mm = timed(lambda: torch.mm(a, b))
    copy_gbs = 2 * src.numel() * 4 / t_copy / 1e9
    gemm_tflops = 2 * 8192 ** 3 / t_mm / 1e12
    del src, dst, a, b
    return {"copy_GBps": round(copy_gbs, 1),
            "copy": "device copy of 512 MiB (bytes read + written per second), best of 5",
            "bf16_gemm_TFLOPs": round(gemm_tflops, 1),
            "gemm": "torch.mm bf16 8192 x 8192 x 8192, contiguous, best of 5"}


def touched_line_bytes(prob, line=128):
    """Bytes of the distinct `line`-byte cache lines the attention's gathers touch (fp8_ds_mla:
    a token's 576 data bytes and its 8 scale bytes lie in different lines of its page)."""
    import numpy as np
    total = 0
    for pool, lists in ((prob.kv, prob.idx_main), (prob.extra_kv, prob.idx_extra)):
        if pool is None or lists is None:
            continue
        P = pool.page_size
        ids = []
        for b in range(prob.T):
            pos = np.asarray(lists[b], dtype=np.int64)
            pos = pos[pos >= 0]
            slots = np.asarray(pool.block_table[b], dtype=np.int64)[pos // P] * P + pos % P
            base = (slots // P) * (P * 584)
            inpg = slots % P
            for lo, n in ((base + inpg * 576, 576), (base + P * 576 + inpg * 8, 8)):
                first, last = lo // line, (lo + n - 1) // line
                span = int((last - first).max()) + 1
                cand = first[:, None] + np.arange(span)[None, :]
                ids.append(cand[cand <= last[:, None]])
        total += np.unique(np.concatenate(ids)).size * line
    return total


def other_configs(dsa, to_device, workloads, torch, dev, flush, names, reps=15, keep=None):
    """Cold per-call latency of the other single-GPU workloads (context beside the headline):
    the fused layer for decode shapes, the attention stage alone for the DSv4 fp8 case.
    keep: a dict that receives the generated problems (for the oracle's timing)."""
    res = {}
    for name in names:
        prob = workloads.make_workload(name)
        if keep is not None:
            keep[name] = prob
        d = to_device(prob, dev)
        T, H = prob.T, prob.H
        out = torch.empty(T, H, prob.d_v, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(T, H, dtype=torch.float32, device=dev)
        if prob.kpool is not None:
            idx = torch.empty(T, prob.topk, dtype=torch.int32, device=dev)
            lens = torch.empty(T, dtype=torch.int32, device=dev)
            ws = dsa.Workspace(dsa.dsa_workspace_size(dsa.ENTRY_DECODE, T=T, n_max=prob.n_max, topk=prob.topk,
                                                      H=H), dev)

            def step():
                dsa.dsa_decode(d.q, d.q_idx, d.w, d.keys, d.kv, d.rows, H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
                               prob.topk, prob.index_scale, prob.softmax_scale, out, lse, idx, lens, ws)
            stage = "layer (scores + top-k + sparse attention)"
            ab = algorithmic_bytes(prob)["total"]
        else:
            n_main = d.idx_main.shape[1]
            n_extra = d.idx_extra.shape[1] if d.idx_extra is not None else 0
            ws = dsa.Workspace(dsa.dsa_workspace_size(dsa.ENTRY_MLA_DECODE, T=T, H=H, n_idx=n_main + n_extra), dev)

            def step():
                dsa.dsa_sparse_mla_decode(d.q, d.kv, d.idx_main, d.extra_kv, d.idx_extra, T, H, prob.d_qk,
                                          prob.d_v, prob.softmax_scale, out, lse, ws)
            stage = "sparse attention over main + extra lists (the stage this case specifies)"
            row_b = {"bf16": 2 * prob.d_qk, "fp8_uniform": prob.d_qk + 4 * prob.d_qk // 64, "fp8_ds_mla": 584}[prob.kv.fmt]
            ab = T * (n_main + n_extra) * (row_b + 4) + T * H * (prob.d_qk * 2 + prob.d_v * 2 + 4)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            flush.sum()
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        us = statistics.median([a.elapsed_time(b) * 1e3 for a, b in evs])
        res[name] = {"stage": stage, "rows": int(T), "context_max": int(prob.n_max), "cold_us": round(us, 2),
                     "algorithmic_bytes": int(ab), "hbm_roofline_frac": round(ab / (HBM_PEAK_GBS * 1e9) / (us * 1e-6), 4)}
        if prob.kv.fmt == "fp8_ds_mla":
            tb = touched_line_bytes(prob) + T * H * (prob.d_qk * 2 + prob.d_v * 2 + 4)
            res[name]["touched_line_bytes"] = int(tb)
            res[name]["touched_line_frac"] = round(tb / (HBM_PEAK_GBS * 1e9) / (us * 1e-6), 4)
            res[name]["touched_note"] = ("distinct 128-byte lines of the gathered rows (576 data bytes and the "
                                         "8 scale bytes of a token sit in different lines) plus q, out and lse")
        del d, out, lse, ws
        torch.cuda.empty_cache()
        log(f"  {name}: {us:.2f} us cold")
    return res


def prefill_chain(dsa, to_device, workloads, torch, dev, reps=3, keep=None):
    """The causal prefill chain (segments 8192 + 1): scores -> top-k -> sparse attention over
    64 heads, each stage timed by its own HIP events; the attention against the bf16 MFMA
    peak (2 * 64 * (576 + 512) FLOP per (row, listed entry)) and the top-k against one read
    of the logits."""
    import numpy as np
    prob = workloads.causal_prefill((8192, 1), name="causal_prefill_8k")
    if keep is not None:
        keep["causal_prefill_8k"] = prob
    d = to_device(prob, dev)
    T = prob.T
    ld = ((prob.n_max + 63) // 64) * 64
    logits = torch.empty(T, ld, dtype=torch.float32, device=dev)
    idx = torch.empty(T, prob.topk, dtype=torch.int32, device=dev)
    lens = torch.empty(T, dtype=torch.int32, device=dev)
    out = torch.empty(T, prob.H, prob.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, prob.H, dtype=torch.float32, device=dev)
    ws = dsa.Workspace(dsa.dsa_workspace_size(dsa.ENTRY_TOPK, T=T, n_max=prob.n_max, topk=prob.topk), dev)

    def run():
        dsa.dsa_index_scores(d.q_idx, d.w, d.keys, d.rows, prob.Hi, prob.di, prob.index_scale, logits)
        dsa.dsa_topk(logits, d.rows, prob.topk, idx, lens, ws)
        dsa.dsa_sparse_mla_prefill(d.q, d.kv, idx, None, None, d.rows, prob.H, prob.d_qk, prob.d_v,
                                   prob.softmax_scale, out, lse)

    run()
    torch.cuda.synchronize()
    dsa.dsa_profile_enable(True)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    prof = dsa.dsa_profile_collect()
    dsa.dsa_profile_enable(False)
    us = {k: round(v["total_ms"] / v["count"] * 1e3, 1) for k, v in prof.items()}
    n = prob.row_len.astype(np.int64)
    visits = int(np.minimum(n, prob.topk).sum())
    att_flop = visits * 2 * prob.H * (prob.d_qk + prob.d_v)
    att_us = us.get("sparse_mla")
    topk_us = sum(v for k, v in us.items() if k.startswith("topk"))
    logit_bytes = int(n.sum()) * 4
    res = {"workload": "causal_prefill_8k (8193 rows, 64 heads x 576/512, indexer 64 x 128, topk 2048)",
           "stages_us": us, "total_us": round(sum(us.values()), 1),
           "attention": {"row_visits": visits, "tflop": round(att_flop / 1e12, 3),
                         "achieved_TFLOPs": round(att_flop / (att_us * 1e-6) / 1e12, 1) if att_us else None,
                         "peak": MFMA_BF16_PEAK_TFLOPS,
                         "frac": round(att_flop / (att_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4) if att_us else None},
           "topk": {"logits_MB": round(logit_bytes / 1e6, 1), "us": round(topk_us, 1),
                    "GBps": round(logit_bytes / (topk_us * 1e-6) / 1e9, 1) if topk_us else None},
           "timing": "HIP events from each dispatch, inputs resident"}
    del d, logits, idx, out, lse, ws
    return res


def attention_backward(dsa, workloads, torch, dev, reps=5):
    """The attention backward (dq and dKV, one list) on 64 rows x 64 heads x 2048 listed rows
    (of 4096-token contexts, bf16 576 rows), after its forward: time, dKV bytes and
    MFMA-equivalent rate. Each row is its own request, so every listed cache row is named once
    and the owner map sends every dKV add to a plain load and store of whole rows. Its cost
    depends on the listed rows, not on the context length."""
    import numpy as np
    from deepseek_sparse_attention_indexer_amd.upload import to_device
    prob = workloads.attention_case(fmt="bf16", B=64, H=64, n_ctx=4096, n_idx=2048, pad="tail", n_pad=0)
    d = to_device(prob, dev)
    T, H = prob.T, prob.H
    out = torch.empty(T, H, prob.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, H, device=dev)
    g = torch.Generator(device="cpu").manual_seed(7)
    dout = torch.randn(T, H, prob.d_v, generator=g).to(torch.bfloat16).to(dev)
    dq = torch.empty(T, H, prob.d_qk, device=dev)
    dkv = torch.zeros(int(d.kv.c.n_slots), prob.d_qk, device=dev)
    dsa.dsa_sparse_mla_prefill(d.q, d.kv, d.idx_main, None, None, d.rows, H, prob.d_qk, prob.d_v,
                               prob.softmax_scale, out, lse)

    ws = dsa.Workspace(dsa.dsa_workspace_size(dsa.ENTRY_MLA_BACKWARD, T=T, H=H, n_idx=int(d.idx_main.shape[1]),
                                              n_slots=int(d.kv.c.n_slots)), dev)

    def run():
        dsa.dsa_sparse_mla_backward(d.q, d.kv, d.idx_main, d.rows, H, prob.d_qk, prob.d_v,
                                    prob.softmax_scale, out, lse, dout, dq, dkv, ws)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    dsa.dsa_profile_enable(True)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    prof = dsa.dsa_profile_collect()
    dsa.dsa_profile_enable(False)
    kernels = {k: round(v["total_ms"] / v["count"] * 1e3, 1) for k, v in prof.items()}
    us = sum(kernels.values())
    pairs = int((np.asarray(prob.idx_main) >= 0).sum())
    flops = pairs * H * 2 * (2 * prob.d_qk + prob.d_v + prob.d_qk + prob.d_v)
    # dKV: one add per (listed entry, column), heads summed first; a row named once is read
    # and written whole (4 + 4 bytes per column)
    dkv_bytes = pairs * prob.d_qk * 8
    dkv_us = kernels.get("sparse_mla_bwd_dkv")
    return {"workload": "attention backward, 64 rows x 64 heads x 2048 of 4096 rows (bf16 576)",
            "kernels_us": kernels, "avg_us": round(us, 1), "gflop": round(flops / 1e9, 2),
            "achieved_tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "dkv_adds": pairs * prob.d_qk, "dkv_bytes": dkv_bytes,
            "dkv_gbps": round(dkv_bytes / (dkv_us * 1e-6) / 1e9, 1) if dkv_us else None,
            "bound": "dKV: the read and write of every listed cache row (HBM); dq/P/dZ: the row gathers",
            "timing": "HIP events from each dispatch, inputs resident"}


def host_cores():
    """The host cores this process may run on (BLAS threads are set to the same count)."""
    return len(os.sched_getaffinity(0))


def cpu_baseline(prob, seconds):
    """The oracle's whole layer for the headline workload, repeated for about `seconds`."""
    import oracle
    from threadpoolctl import threadpool_limits
    cores = host_cores()
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.layer_row(prob, 0)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    us = el / reps * 1e6
    return {"value": round(us, 1), "unit": "us", "cores": int(cores), "kind": "oracle",
            "sample": f"the whole layer of the same workload (fp64 scores of all {int(prob.row_len[0])} "
                      f"candidates, stable top-{prob.topk}, attention), repeated {reps}x in {el:.1f} s"}


def cpu_oracle_configs(probs, sample_rows=512):
    """The oracle (numpy fp64, all host cores) on the other workloads: the tiny, 32k and 1M
    decode layers and the DSv4 attention stage whole; the causal prefill on a seeded stratified
    sample of rows (rows 0, 2046, 2047, 8191 and the 1-token segment among them), its time per
    row scaled to all rows and labelled extrapolated."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    cores = host_cores()
    res = {}
    with threadpool_limits(limits=cores):
        for name in ("tiny_decode", "glm_decode_32k", "long_decode_1m"):
            if name not in probs:
                continue
            prob = probs[name]
            t0 = time.perf_counter()
            for t in range(prob.T):
                oracle.layer_row(prob, t)
            el = time.perf_counter() - t0
            res[name] = {"us": round(el * 1e6, 1), "rows": int(prob.T), "what": "whole layer (scores, top-k, attention)"}
        if "dsv4_fp8_decode" in probs:
            prob = probs["dsv4_fp8_decode"]
            t0 = time.perf_counter()
            for t in range(prob.T):
                oracle.attention_row(prob, t, prob.idx_main[t], prob.idx_extra[t])
            el = time.perf_counter() - t0
            res["dsv4_fp8_decode"] = {"us": round(el * 1e6, 1), "rows": int(prob.T),
                                      "what": "whole attention stage (main + extra lists)"}
        if "causal_prefill_8k" in probs:
            prob = probs["causal_prefill_8k"]
            seg = int(prob.row_len[prob.T - 2])
            rng = np.random.default_rng(11)
            fixed = [0, 2046, 2047, seg - 1, prob.T - 1]
            edges = np.linspace(0, seg, sample_rows - len(fixed) + 1).astype(int)
            rows = sorted(set(fixed) | {int(rng.integers(lo, hi)) for lo, hi in zip(edges[:-1], edges[1:]) if hi > lo})
            t0 = time.perf_counter()
            for t in rows:
                oracle.layer_row(prob, t)
            el = time.perf_counter() - t0
            res["causal_prefill_8k"] = {"us": round(el / len(rows) * prob.T * 1e6, 1), "rows": int(prob.T),
                                        "sampled_rows": len(rows), "sample_s": round(el, 2),
                                        "what": "whole layer per row on a stratified sample, scaled to all rows: "
                                                "extrapolated"}
    return {"cores": cores, "configs": res}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="glm_decode_128k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill indexer measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the attention backward measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (32k, 1M fp8-key decode, DSv4 fp8 attention, multi-token)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured copy / GEMM ceilings (e.g. under counter passes)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--attn-plan", default=None, metavar="HT,SPLITS",
                    help="force the attention launch plan (head tiles per workgroup, splits per row; "
                         "dsa_launch_override) instead of the library's table, for plan sweeps")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU hot path only: the library runs the layer on one "
              "GPU's share (heads or a slice of the candidates), with no collectives", file=sys.stderr)
        sys.exit(2)

    import torch
    import deepseek_sparse_attention_indexer_amd as dsa
    from deepseek_sparse_attention_indexer_amd.upload import to_device
    import workloads

    plan = None
    if args.attn_plan:
        ht, sp = (int(v) for v in args.attn_plan.split(","))
        dsa.dsa_launch_override(head_tiles=ht, n_split=sp)
        plan = f"{ht} head tiles x {sp} splits (forced)"
    prob = workloads.make_workload(args.workload)
    if prob.kpool is None:
        raise SystemExit("bench.py times the whole layer: pick a workload with an indexer")
    dev = torch.device("cuda:0")
    d = to_device(prob, dev)
    T, H = prob.T, prob.H
    out = torch.empty(T, H, prob.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, H, dtype=torch.float32, device=dev)
    idx = torch.empty(T, prob.topk, dtype=torch.int32, device=dev)
    lens = torch.empty(T, dtype=torch.int32, device=dev)
    ws = dsa.Workspace(dsa.dsa_workspace_size(dsa.ENTRY_DECODE, T=T, n_max=prob.n_max, topk=prob.topk, H=H), dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)    # 1 GiB

    def step():
        dsa.dsa_decode(d.q, d.q_idx, d.w, d.keys, d.kv, d.rows, H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
                       prob.topk, prob.index_scale, prob.softmax_scale, out, lse, idx, lens, ws)

    def evict():
        flush.sum()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K cold steps, each bracketed by events, eviction outside the events
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        evict()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cold_us = [a.elapsed_time(b) * 1e3 for a, b in evs]
    cold = statistics.median(cold_us)

    # ---- warm: back to back
    wa, wb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wa.record()
    for _ in range(K):
        step()
    wb.record()
    torch.cuda.synchronize()
    warm = wa.elapsed_time(wb) * 1e3 / K

    # ---- per-kernel durations (events around each launch, cold steps again)
    dsa.dsa_profile_enable(True)
    for _ in range(K):
        evict()
        step()
    torch.cuda.synchronize()
    prof = dsa.dsa_profile_collect()
    dsa.dsa_profile_enable(False)
    per_kernel = {k: round(v["total_ms"] / v["count"] * 1e3, 2) for k, v in prof.items()}
    dom = max(prof, key=lambda k: prof[k]["total_ms"] / prof[k]["count"])
    dom_us = prof[dom]["total_ms"] / prof[dom]["count"] * 1e3
    dom_bytes = kernel_bytes(prob, dom)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9 if dom_bytes else None
    traffic = read_traffic(dom, args.workload)
    # the same per-dispatch timing of a trivial library kernel (one 576-wide bf16 row written
    # into a one-row cache): the fixed cost every launch carries on this system
    row = torch.zeros(1, prob.d_qk, dtype=torch.bfloat16, device=dev)
    one = dsa.KVCache("bf16", torch.zeros(1, prob.d_qk, dtype=torch.bfloat16, device=dev), prob.kv.d_nope,
                      prob.kv.d_rope)
    slot0 = torch.zeros(1, dtype=torch.int32, device=dev)
    dsa.dsa_profile_enable(True)
    for _ in range(K):
        dsa.dsa_kv_cache_write(row, slot0, one)
    torch.cuda.synchronize()
    prof_f = dsa.dsa_profile_collect()
    dsa.dsa_profile_enable(False)
    floor_us = prof_f["cache_write_kv"]["total_ms"] / prof_f["cache_write_kv"]["count"] * 1e3

    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    ab = algorithmic_bytes(prob)
    layer_frac = (ab["total"] / (HBM_PEAK_GBS * 1e9)) / (cold * 1e-6)

    res = {
        "metric": "DSA layer µs (scores+topk+sparse attn) at 128k decode; % HBM roofline",
        "value": round(cold, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(cold / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(cold / PAGE_128K_DECODE_US, 4) if args.workload == "glm_decode_128k" else None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": T, "context": int(prob.row_len.max()),
                   "heads": H, "d_qk": prob.d_qk, "d_v": prob.d_v, "indexer": f"{prob.Hi}x{prob.di} {prob.kpool.dtype}",
                   "topk": prob.topk, "kv_cache": f"{prob.kv.fmt} paged {prob.kv.page_size} shuffled",
                   "cache_state": "cold: 1 GiB read evicts L2 + MALL before each step",
                   **({"attn_plan": plan} if plan else {})},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1) if achieved else None,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                     "traffic": traffic, "kernel_algorithmic_bytes": dom_bytes, "avg_us": round(dom_us, 2),
                     "timing": "HIP events around each launch on the launch stream, cold steps",
                     "dispatch_floor_us": round(floor_us, 2),
                     "frac_net_of_dispatch_floor": round(dom_bytes / ((dom_us - floor_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                     if dom_bytes and dom_us > floor_us else None,
                     "floor_note": "dispatch_floor_us: the same per-dispatch event timing of a trivial library kernel "
                                   "(one row written into a one-row cache); frac_net_of_dispatch_floor divides by "
                                   "avg_us minus that floor "
                                   "(context only; frac is the measured one)"},
        "layer": {"algorithmic_bytes": ab, "hbm_roofline_frac": round(layer_frac, 4),
                  "warm_us": round(warm, 2), "cold_us_p10_p90": [round(sorted(cold_us)[K // 10], 2),
                                                                  round(sorted(cold_us)[(9 * K) // 10], 2)],
                  "per_kernel_us": per_kernel, "kernel_sum_us": round(sum(per_kernel.values()), 2),
                  "gap_us": round(cold - sum(per_kernel.values()), 2),
                  "gap_note": "layer time minus the sum of its kernels' own durations: launch and "
                              "inter-kernel idle time of the dependent kernels on one stream",
                  "timed_wall_s": round(wall, 4)},
        "vs_baseline_note": "value / 411 us: the pages' Gluon 128k decode total (tokenspeed PR 627, "
                            "GFX9-class GPU, heads and precision unstated); context, not the target",
    }
    cal = None
    if not args.no_ceilings:
        log("measured ceilings ...")
        cal = calibration(torch, dev)
        cal["layer_frac_of_copy"] = round((ab["total"] / (cal["copy_GBps"] * 1e9)) / (cold * 1e-6), 4)
        if achieved:
            cal["roofline_kernel_frac_of_copy"] = round(achieved / cal["copy_GBps"], 4)
        res["measured_ceilings"] = cal
    if not args.no_prefill:
        log("prefill indexer ...")
        res["prefill_indexer"] = pf = prefill_indexer(dsa, to_device, workloads, torch, dev)
        if cal:
            pf["frac_of_measured_gemm"] = round(pf["achieved"] / cal["bf16_gemm_TFLOPs"], 4)
    kept = {}
    if not args.no_prefill:
        log("prefill chain ...")
        res["prefill_chain"] = prefill_chain(dsa, to_device, workloads, torch, dev, keep=kept)
        if cal and res["prefill_chain"]["attention"]["achieved_TFLOPs"]:
            res["prefill_chain"]["attention"]["frac_of_measured_gemm"] = round(
                res["prefill_chain"]["attention"]["achieved_TFLOPs"] / cal["bf16_gemm_TFLOPs"], 4)
    if not args.no_backward:
        log("attention backward ...")
        res["attention_backward"] = attention_backward(dsa, workloads, torch, dev)
    if not args.no_configs:
        log("other workloads ...")
        res["other_configs"] = other_configs(dsa, to_device, workloads, torch, dev, flush,
                                             ["tiny_decode", "glm_decode_32k", "long_decode_1m", "dsv4_fp8_decode",
                                              "spec_decode_b16_q4_32k", "extend_64_128k"], keep=kept)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(prob, args.cpu_seconds)
        if kept:
            res["cpu_oracle_configs"] = cpu_oracle_configs(kept)
    log(f"cold {cold:.2f} us  warm {warm:.2f} us  per-kernel {per_kernel}  wall {wall:.3f} s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
