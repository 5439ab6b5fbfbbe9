"""The boundary's contract on the GPU, beyond per-value parity:

* caches larger than 4 GiB: listed rows and key pages placed past the 2 GiB and 4 GiB byte
  offsets (and straddling them) are read correctly (64-bit addressing of every gather);
* the fused decode captured once in a HIP graph and replayed with new inputs in place gives
  exactly the eager results (the workspace's control words stay zero at rest; no memset node);
* every forward entry gives bit-identical results when run twice on the same inputs;
* DSA_LOG=1 prints one line per kernel launch with the launch row that chose it, and nothing
  without it.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import attention_ok, scores_ok, topk_ok
from dev import dsa, need_gpu, run_attention, say, upload, workload

pytestmark = [pytest.mark.gpu, need_gpu]

GiB = 1 << 30


# --------------------------------------------------------------------------- caches past 4 GiB

def _far_pages(n_need, page_bytes, n_big, seed):
    """n_need distinct page ids of an n_big-page cache: the pages that straddle and follow the
    2 GiB and 4 GiB byte offsets, the last page, then random pages past 2 GiB."""
    fixed = []
    for edge in (2 * GiB, 4 * GiB):
        p = edge // page_bytes
        fixed += [p, p + 1] if edge % page_bytes else [p - 1, p]
    fixed.append(n_big - 1)
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(2 * GiB // page_bytes + 2, n_big - 1), fixed)
    rest = rng.choice(pool, size=max(0, n_need - len(fixed)), replace=False)
    pages = np.concatenate([np.asarray(fixed[:n_need]), rest]).astype(np.int64)
    rng.shuffle(pages)
    return pages


def _relocate(pages_dev, bt, page_bytes, min_bytes, seed):
    """A cache of at least min_bytes whose pages, for every used entry of the block table bt
    [n_req, w] (numpy), hold the content of pages_dev[bt[b, lp]], moved to far page ids.
    pages_dev: device tensor [n_pages, page_elems]. Returns (big device tensor, new table)."""
    used = sorted(set(bt.ravel().tolist()))
    n_big = -(-min_bytes // page_bytes)
    far = _far_pages(len(used), page_bytes, n_big, seed)
    remap = dict(zip(used, far.tolist()))
    big = torch.zeros((n_big,) + tuple(pages_dev.shape[1:]), dtype=pages_dev.dtype, device="cuda")
    src = torch.as_tensor(used, device="cuda")
    dst = torch.as_tensor([remap[u] for u in used], device="cuda")
    big[dst] = pages_dev[src]
    new_bt = np.vectorize(remap.get)(bt).astype(np.int32)
    starts = np.array(sorted(remap.values())) * page_bytes
    # pages at and around both offsets (a page straddles an offset unless it divides the page)
    assert (starts >= 4 * GiB).any() and ((starts + page_bytes > 2 * GiB) & (starts <= 2 * GiB)).any()
    return big, new_bt


def test_decode_with_caches_past_4_gib():
    """The fused layer (scores -> top-k -> attention) on a bf16 key cache and a bf16 latent
    cache of more than 5 GiB each, with the requests' pages moved past the 2 and 4 GiB offsets;
    compared with the oracle on the original (small) caches."""
    m = dsa()
    prob = workload("glm_decode", n_ctx=3000, B=2, ctx_lens=(3000, 2100), topk=512, H=64)
    d = upload(prob)
    P = prob.kv.page_size
    kv_pages = d.kv.keep[0].view(-1, P * prob.d_qk)                 # bf16 [pages, 64 * 576]
    key_pages = d.keys.keep[0].view(-1, P * prob.di)                # bf16 [pages, 64 * 128]
    kv_big, kv_bt = _relocate(kv_pages, prob.kv.block_table, P * prob.d_qk * 2, 5 * GiB + 12345, 1)
    key_big, key_bt = _relocate(key_pages, prob.kpool.block_table, P * prob.di * 2, 5 * GiB + 777, 2)
    say("decode with caches of", kv_big.numel() * 2 / GiB, "and", key_big.numel() * 2 / GiB, "GiB")
    kv = m.KVCache("bf16", kv_big.view(-1, prob.d_qk), prob.kv.d_nope, prob.kv.d_rope, page_size=P,
                   block_table=torch.from_numpy(kv_bt).cuda())
    keys = m.KeyCache(key_big.view(-1, prob.di), page_size=P, block_table=torch.from_numpy(key_bt).cuda())
    T, H = prob.T, prob.H
    out = torch.full((T, H, prob.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), device="cuda")
    idx = torch.full((T, prob.topk), -7, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_DECODE, T=T, n_max=prob.n_max, topk=prob.topk, H=H))
    m.dsa_decode(d.q, d.q_idx, d.w, keys, kv, d.rows, H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
                 prob.topk, prob.index_scale, prob.softmax_scale, out, lse, idx, lens, ws)
    logits = torch.full((T, prob.n_max), float("nan"), device="cuda")
    m.dsa_index_scores(d.q_idx, d.w, keys, d.rows, prob.Hi, prob.di, prob.index_scale, logits)
    torch.cuda.synchronize()
    out, lse, idx, lens = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), lens.cpu().numpy()
    logits = logits.cpu().numpy()
    del kv_big, key_big, kv, keys
    torch.cuda.empty_cache()
    for t in range(T):
        n = int(prob.row_len[t])
        scores = oracle.index_scores_row(prob, t)
        ok, msg = scores_ok(logits[t, :n], scores)
        assert ok, f"row {t}: scores {msg}"
        ok, msg = topk_ok(scores, prob.topk, idx[t], lens[t])
        assert ok, f"row {t}: top-k {msg}"
        o_ref, l_ref = oracle.attention_row(prob, t, idx[t])
        ok, msg = attention_ok(out[t], lse[t], o_ref, l_ref, "bf16")
        assert ok, f"row {t}: attention {msg}"


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_fp8_ds_mla_attention_with_a_cache_past_4_gib(mode):
    """Two-list fp8_ds_mla attention (584-byte tokens in page-planar 256-token pages: data and
    scale bytes of one token are 147 KiB apart) with both caches above 5 GiB and their pages
    past the 2 and 4 GiB offsets."""
    m = dsa()
    prob = workload("attention_case", fmt="fp8_ds_mla", B=3, H=16, n_ctx=2000, n_idx=128, page_size=256,
                    n_extra=300, pad="shuffled", n_pad=9)
    d = upload(prob)
    pb = prob.kv.page_size * 584
    main_big, main_bt = _relocate(d.kv.keep[0], prob.kv.block_table, pb, 5 * GiB + 1, 3)
    extra_big, extra_bt = _relocate(d.extra_kv.keep[0], prob.extra_kv.block_table, pb, 5 * GiB + 3, 4)
    say("fp8_ds_mla attention with caches of", main_big.numel() / GiB, "GiB", mode)
    kv = m.KVCache("fp8_ds_mla", main_big, 448, 64, page_size=256, block_table=torch.from_numpy(main_bt).cuda())
    ekv = m.KVCache("fp8_ds_mla", extra_big, 448, 64, page_size=256, block_table=torch.from_numpy(extra_bt).cuda())
    d.kv, d.extra_kv = kv, ekv
    out, lse = run_attention(prob, d=d, mode=mode)
    del main_big, extra_big, kv, ekv, d
    torch.cuda.empty_cache()
    for t in range(prob.T):
        o_ref, l_ref = oracle.attention_row(prob, t, prob.idx_main[t], prob.idx_extra[t])
        ok, msg = attention_ok(out[t], lse[t], o_ref, l_ref, "fp8_ds_mla")
        assert ok, f"row {t}: {msg}"


# --------------------------------------------------------------------------- HIP graph capture

def _decode_buffers(prob, d):
    T, H = prob.T, prob.H
    return dict(out=torch.zeros((T, H, prob.d_v), dtype=torch.bfloat16, device="cuda"),
                lse=torch.zeros((T, H), device="cuda"),
                idx=torch.zeros((T, prob.topk), dtype=torch.int32, device="cuda"),
                lens=torch.zeros((T,), dtype=torch.int32, device="cuda"))


def _decode_call(m, prob, d, b, ws):
    m.dsa_decode(d.q, d.q_idx, d.w, d.keys, d.kv, d.rows, prob.H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
                 prob.topk, prob.index_scale, prob.softmax_scale, b["out"], b["lse"], b["idx"], b["lens"], ws)


def _snap(b):
    return {k: v.clone() for k, v in b.items()}


def _same(a, b):
    return all(torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k]) for k in a)


@pytest.mark.parametrize("label,kw", [
    ("ragged_20k_b3", dict(n_ctx=20000, B=3, ctx_lens=(20000, 700, 17001))),
    ("glm_128k", dict(n_ctx=131072)),
], ids=["ragged_20k_b3", "glm_128k"])
def test_decode_graph_replay_matches_eager(label, kw):
    """dsa_decode captured once in a HIP graph (workspace initialised before the capture) and
    replayed with the step's inputs (q, q_idx, w) rewritten in place between replays; every
    replay equals the eager call on the same inputs bit for bit. Eager work runs between the
    replays, as in a serving loop."""
    m = dsa()
    prob = workload("glm_decode", **kw)
    alt = workload("glm_decode", seed=5, **kw)
    d = upload(prob)
    inputs = {"A": (d.q.clone(), d.q_idx.clone(), d.w.clone())}
    da = upload(alt)
    inputs["B"] = (da.q.clone(), da.q_idx.clone(), da.w.clone())
    del da

    def load(name):
        q, qi, w = inputs[name]
        d.q.copy_(q)
        d.q_idx.copy_(qi)
        d.w.copy_(w)

    ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_DECODE, T=prob.T, n_max=prob.n_max, topk=prob.topk, H=prob.H))
    buf = _decode_buffers(prob, d)
    eager = {}
    for name in ("A", "B"):
        load(name)
        _decode_call(m, prob, d, buf, ws)
        torch.cuda.synchronize()
        eager[name] = _snap(buf)
    assert not _same(eager["A"], eager["B"])
    load("A")
    torch.cuda.synchronize()
    say("graph capture", label)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm the side stream, as torch asks before capture
        _decode_call(m, prob, d, buf, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decode_call(m, prob, d, buf, ws)
    torch.cuda.synchronize()
    for rep, name in enumerate(("A", "B", "B", "A", "B")):
        load(name)
        for v in buf.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_snap(buf), eager[name]), f"replay {rep} ({name}) differs from the eager call"
        # eager work between replays: an eager decode of the other inputs on a fresh workspace
        other = "B" if name == "A" else "A"
        load(other)
        ws2 = m.Workspace(ws.nbytes)
        b2 = _decode_buffers(prob, d)
        _decode_call(m, prob, d, b2, ws2)
        torch.cuda.synchronize()
        assert _same(_snap(b2), eager[other])
    del g


# --------------------------------------------------------------------------- run twice

def _twice(fn):
    a = fn()
    torch.cuda.synchronize()
    a = [x.clone() for x in a]
    b = fn()
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        xi = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
        yi = y.view(torch.int16) if y.dtype == torch.bfloat16 else y
        assert torch.equal(xi, yi)
    return a


@pytest.mark.parametrize("label,kw", [
    ("glm_32k", dict(n_ctx=32768)),
    ("spec_b4_q4_h64", dict(n_ctx=6000, B=4, q_len=4, ctx_lens=(6000, 5001, 2100, 4444))),
    ("extend_64_20k_h16", dict(n_ctx=20000, q_len=64, H=16)),
], ids=["glm_32k", "spec_b4_q4_h64", "extend_64_20k_h16"])
def test_forward_entries_are_deterministic(label, kw):
    """Scores, top-k (indices in the same order), the fused decode, and both attention entries,
    each called twice on one workspace: bit-identical results."""
    m = dsa()
    prob = workload("glm_decode", **kw)
    d = upload(prob)
    say("run twice", label)
    T, H = prob.T, prob.H
    logits = torch.empty((T, prob.n_max), device="cuda")
    ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_DECODE, T=T, n_max=prob.n_max, topk=prob.topk, H=H))

    def scores():
        m.dsa_index_scores(d.q_idx, d.w, d.keys, d.rows, prob.Hi, prob.di, prob.index_scale, logits)
        return [logits]
    _twice(scores)
    idx = torch.empty((T, prob.topk), dtype=torch.int32, device="cuda")
    lens = torch.empty((T,), dtype=torch.int32, device="cuda")

    def topk():
        m.dsa_topk(logits, d.rows, prob.topk, idx, lens, ws)
        return [idx, lens]
    _twice(topk)
    buf = _decode_buffers(prob, d)

    def decode():
        _decode_call(m, prob, d, buf, ws)
        return list(buf.values())
    _twice(decode)
    out = torch.empty((T, H, prob.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), device="cuda")

    def mla_decode():
        m.dsa_sparse_mla_decode(d.q, d.kv, idx, None, None, T, H, prob.d_qk, prob.d_v, prob.softmax_scale,
                                out, lse, ws)
        return [out, lse]
    if prob.T == prob.n_req:                      # the decode entry takes row t as request t
        _twice(mla_decode)

    def mla_prefill():
        m.dsa_sparse_mla_prefill(d.q, d.kv, idx, None, None, d.rows, H, prob.d_qk, prob.d_v,
                                 prob.softmax_scale, out, lse)
        return [out, lse]
    _twice(mla_prefill)


def test_attention_two_lists_fp8_deterministic():
    """The split-KV decode entry over two fp8_ds_mla lists (DeepSeek-V4 shape, 64 requests)."""
    m = dsa()
    prob = workload("attention_case", fmt="fp8_ds_mla", B=16, H=64, n_ctx=5000, n_idx=1000, page_size=64,
                    n_extra=230, pad="tail", n_pad=7)
    d = upload(prob)
    out = torch.empty((prob.T, prob.H, prob.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((prob.T, prob.H), device="cuda")
    ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_MLA_DECODE, T=prob.T, H=prob.H, n_idx=1230))

    def run():
        m.dsa_sparse_mla_decode(d.q, d.kv, d.idx_main, d.extra_kv, d.idx_extra, prob.T, prob.H, prob.d_qk,
                                prob.d_v, prob.softmax_scale, out, lse, ws)
        return [out, lse]
    _twice(run)


# --------------------------------------------------------------------------- launch log

_LOG_CHILD = """
import sys
sys.path.insert(0, {tests!r})
sys.path.insert(0, {root!r})
import torch
from dev import run_decode, workload
run_decode(workload("tiny_decode"))
torch.cuda.synchronize()
print("child done", flush=True)
"""


@pytest.mark.parametrize("log", ["1", None])
def test_dsa_log_prints_the_launch_rows(log):
    """DSA_LOG is read once per process, so each setting runs the tiny decode in a child."""
    here = os.path.dirname(os.path.abspath(__file__))
    code = _LOG_CHILD.format(tests=here, root=os.path.dirname(here))
    env = {k: v for k, v in os.environ.items() if k != "DSA_LOG"}
    if log:
        env["DSA_LOG"] = log
    say(f"DSA_LOG={log}: tiny decode in a child process")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "child done" in r.stdout, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[dsa] ")]
    if not log:
        assert lines == []
        return
    kernels = [ln.split()[1] for ln in lines]
    assert kernels == ["index_scores", "topk_lds", "sparse_mla", "mla_combine"], lines
    assert "T=1 n_max=512 Hi=4 di=64" in lines[0], lines[0]
    assert "topk=128" in lines[1] and "in registers" in lines[1], lines[1]
    assert "H=16 (padded 16) list 128+0" in lines[2] and "decode" in lines[2], lines[2]
    assert "split(s)" in lines[3], lines[3]
