"""The whole layer on the GPU: the fused dsa_decode entry, and the prefill chain
dsa_index_scores -> dsa_topk -> dsa_sparse_mla_prefill, against the oracle.

Top-k is checked with rule T against the oracle's fp64 scores; attention is checked against
the oracle run on the GPU's own selection (so near-tie choices do not leak into it)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.compare import attention_ok, scores_ok, topk_ok
from dev import dsa, need_gpu, run_decode, run_scores, say, upload, workload

pytestmark = [pytest.mark.gpu, need_gpu]

DECODE = [
    ("tiny", "tiny_decode", dict()),
    ("ragged_b3", "glm_decode", dict(n_ctx=3000, B=3, ctx_lens=(3000, 1, 777), topk=256)),
    ("glm_32k", "glm_decode", dict(n_ctx=32768)),
    ("glm_128k", "glm_decode", dict(n_ctx=131072)),
    ("long_1m_fp8_keys", "long_decode", dict()),
    ("b4_20k_long_rows", "glm_decode", dict(n_ctx=20000, B=4, ctx_lens=(20000, 17000, 100, 19999), H=16)),
    # several query tokens per request (causal among themselves): speculative verification
    # and an extend chunk; the 96-row case scores with the shared-key kernel
    ("spec_b3_q4", "glm_decode", dict(n_ctx=20000, B=3, q_len=4, ctx_lens=(20000, 17001, 900), H=16)),
    ("extend_64_20k", "glm_decode", dict(n_ctx=20000, q_len=64, H=16)),
    ("spec_b24_q4", "glm_decode", dict(n_ctx=9000, B=24, q_len=4, H=16, topk=512)),
    # 16 rows x 64 heads: the attention shares each gathered block among all 64 heads (8-wave
    # workgroups), with splits
    ("spec_b4_q4_h64", "glm_decode", dict(n_ctx=6000, B=4, q_len=4, ctx_lens=(6000, 5001, 2100, 4444))),
    # the TP=8 share of a 64-head model: 8 attention heads
    ("glm_128k_h8", "glm_decode", dict(n_ctx=131072, H=8)),
]


@pytest.mark.parametrize("label,name,kw", DECODE, ids=[d[0] for d in DECODE])
def test_fused_decode(label, name, kw):
    prob = workload(name, **kw)
    say("decode", label)
    out, lse, idx, lens = run_decode(prob)
    for t in range(prob.T):
        scores = oracle.index_scores_row(prob, t)
        ok, msg = topk_ok(scores, prob.topk, idx[t], lens[t])
        assert ok, f"row {t}: top-k {msg}"
        o_ref, l_ref = oracle.attention_row(prob, t, idx[t])
        ok, msg = attention_ok(out[t], lse[t], o_ref, l_ref, prob.kv.fmt)
        assert ok, f"row {t}: attention {msg}"


@pytest.mark.parametrize("log2", [False, True], ids=["ln", "log2"])
def test_fused_decode_with_sinks(log2):
    """The fused entry with DeepSeek-V4's attention options: per-head sinks in the softmax
    denominator and the lse in either base (split-KV path: 64 heads over 2048 rows)."""
    import dataclasses
    from workloads.gen import sinks
    base = workload("glm_decode", n_ctx=20000, B=2, ctx_lens=(20000, 700), topk=2048)
    prob = dataclasses.replace(base, sink=sinks(0, base.H), lse_log2=log2)
    say("decode sinks", "log2" if log2 else "ln")
    out, lse, idx, lens = run_decode(prob)
    for t in range(prob.T):
        o_ref, l_ref = oracle.attention_row(prob, t, idx[t])
        ok, msg = attention_ok(out[t], lse[t], o_ref, l_ref, prob.kv.fmt)
        assert ok, f"row {t}: attention {msg}"


def _prefill_chain(prob):
    m = dsa()
    d = upload(prob)
    logits = run_scores(prob, d, ld_pad=0)
    idx = torch.full((prob.T, prob.topk), -7, dtype=torch.int32, device="cuda")
    lens = torch.full((prob.T,), -7, dtype=torch.int32, device="cuda")
    ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_TOPK, T=prob.T, n_max=prob.n_max, topk=prob.topk))
    m.dsa_topk(logits, d.rows, prob.topk, idx, lens, ws)
    out = torch.full((prob.T, prob.H, prob.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((prob.T, prob.H), float("nan"), device="cuda")
    m.dsa_sparse_mla_prefill(d.q, d.kv, idx, None, None, d.rows, prob.H, prob.d_qk, prob.d_v,
                             prob.softmax_scale, out, lse)
    torch.cuda.synchronize()
    return (logits.cpu().numpy(), idx.cpu().numpy(), lens.cpu().numpy(), out.float().cpu().numpy(),
            lse.cpu().numpy())


def _check_prefill_rows(prob, res, rows):
    logits, idx, lens, out, lse = res
    for t in rows:
        n = int(prob.row_len[t])
        scores = oracle.index_scores_row(prob, t)
        ok, msg = scores_ok(logits[t, :n], scores)
        assert ok, f"row {t}: scores {msg}"
        ok, msg = topk_ok(scores, prob.topk, idx[t], lens[t])
        assert ok, f"row {t}: top-k {msg}"
        o_ref, l_ref = oracle.attention_row(prob, t, idx[t])
        ok, msg = attention_ok(out[t], lse[t], o_ref, l_ref, "bf16")
        assert ok, f"row {t}: attention {msg}"


def test_prefill_chain_small_all_rows():
    prob = workload("causal_prefill", seg_lens=(300, 1, 45), topk=64, H=32)
    say("prefill chain small")
    _check_prefill_rows(prob, _prefill_chain(prob), range(prob.T))


def _prefill_sample(prob, n=256, seed=7):
    """A seeded stratified sample of the causal prefill's rows: one row from each of n - 24
    equal strata of the 8192-token segment, plus fixed rows: the first, every row 2040..2055
    (where the -1 padding ends at topk 2048), the last of the segment and the 1-token segment."""
    fixed = [0, 1, 2, 63, 64] + list(range(2040, 2056)) + [4096, 8191, prob.T - 1]
    seg = int(prob.row_len[prob.T - 2])                        # the long segment's length
    rng = np.random.default_rng(seed)
    edges = np.linspace(0, seg, n - len(fixed) + 1).astype(int)
    strat = [int(rng.integers(lo, hi)) for lo, hi in zip(edges[:-1], edges[1:]) if hi > lo]
    rows = sorted(set(fixed) | set(strat))
    assert len(rows) >= n - 8
    return rows


def test_prefill_chain_full_size():
    """One 8192-token segment plus a 1-token segment, topk 2048 with -1 padding for the first
    2047 rows. Every row: the top-k set equals the oracle's stable top-k of the GPU's own fp32
    logits exactly (the selection is integer work on the same scores), lens and the -1 tail.
    A stratified sample of 256 rows: scores against the fp64 oracle, rule T against the
    oracle's fp64 scores, attention against the oracle on the GPU's selection."""
    prob = workload("causal_prefill", seg_lens=(8192, 1))
    say("prefill chain 8193 rows")
    res = _prefill_chain(prob)
    logits, idx, lens, out, _ = res
    exp_lens = np.minimum(prob.row_len, prob.topk)
    assert np.array_equal(lens, exp_lens)
    assert np.isfinite(out).all()
    for t in range(prob.T):
        n = int(prob.row_len[t])
        m = int(exp_lens[t])
        ref_idx, m_ref = oracle.topk_row(logits[t, :n].astype(np.float64), prob.topk)
        assert m_ref == m
        assert np.all(idx[t, m:] == -1), f"row {t}: padding"
        got = idx[t, :m]
        assert np.unique(got).size == m, f"row {t}: duplicates"
        assert set(got.tolist()) == set(ref_idx[:m].tolist()), f"row {t}: set differs from the exact top-k of its logits"
    rows = _prefill_sample(prob)
    say(f"  all {prob.T} top-k sets exact; {len(rows)} sampled rows against the oracle")
    _check_prefill_rows(prob, res, rows)
    # the 1-token segment attends to its own row only
    row = oracle.kv_rows(prob.kv, 1, np.array([0]))[0]
    assert np.abs(out[8192] - row[None, :512]).max() < 2e-2
