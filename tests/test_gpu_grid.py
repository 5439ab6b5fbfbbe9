"""The prefill correctness grid of radixark/miles PR 3608 (section "Correctness": forward and
backward against a full-precision reference over 5 head counts x 6 topk x {packed, 1-token
segments, causal, batch 2} x {tail, shuffled} padding), at small sizes, on the prefill entry.

Head counts 8, 16, 32, 64 and 128 (8 and 16 are the TP-local shares at TP = 8 and 4 of a 64-head
model); topk 32, 64, 96, 128, 160, 256 (96 and 160 give three and five 32-row blocks: one more
than the two-block ring, the count the same PR's "What" section names as a stale-stage hazard).
Per case: the forward over every row, sampled rows against the oracle (attention_ok); the
backward over the sampled rows, fed the oracle's forward (out rounded to bf16, lse to fp32),
against the oracle's gradient at those outputs (dq and dkv within 2%, as in test_gpu_backward).
"""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import attention_ok
from workloads.gen import GRID_LAYOUTS, grid_base, grid_lists
from dev import dsa, need_gpu, run_backward, say, upload
from test_gpu_backward import _check as check_backward, _oracle_forward

pytestmark = [pytest.mark.gpu, need_gpu]

HEADS = (8, 16, 32, 64, 128)
TOPKS = (32, 64, 96, 128, 160, 256)
PADS = ("tail", "shuffled")


@functools.lru_cache(maxsize=2)
def _base(layout, H):
    return grid_base(layout, H, seed=H)


def _sample(T, topk, seed):
    rng = np.random.default_rng(seed)
    fixed = {0, T - 1, min(topk - 1, T - 1), min(topk, T - 1)}
    rest = rng.choice(T, size=min(T, 10), replace=False).tolist()
    return sorted(fixed | set(rest))[:12]


def _forward(prob, d, idx_dev):
    m = dsa()
    out = torch.full((prob.T, prob.H, prob.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((prob.T, prob.H), float("nan"), device="cuda")
    m.dsa_sparse_mla_prefill(d.q, d.kv, idx_dev, None, None, d.rows, prob.H, prob.d_qk, prob.d_v,
                             prob.softmax_scale, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("layout", list(GRID_LAYOUTS))
@pytest.mark.parametrize("H", HEADS)
def test_prefill_grid(H, layout):
    base = _base(layout, H)
    d = upload(base)
    n_fail = []
    for topk in TOPKS:
        for pad in PADS:
            idx = grid_lists(base, topk, pad, seed=topk + (pad == "shuffled"))
            prob = dataclasses.replace(base, topk=topk, idx_main=idx)
            say(f"grid H={H} {layout} topk={topk} {pad}")
            out, lse = _forward(prob, d, torch.from_numpy(idx).cuda())
            assert np.isfinite(out).all()
            rows = _sample(prob.T, topk, seed=H * 1000 + topk)
            for t in rows:
                o_ref, l_ref = oracle.attention_row(prob, t, idx[t])
                ok, msg = attention_ok(out[t], lse[t], o_ref, l_ref, "bf16")
                assert ok, f"H={H} {layout} topk={topk} {pad} row {t}: forward {msg}"
            # backward on the sampled rows (their own problem, so the dkv sum is theirs alone)
            sub = dataclasses.replace(prob, T=len(rows), q=prob.q[rows], row_req=prob.row_req[rows],
                                      row_len=prob.row_len[rows], idx_main=idx[rows])
            rng = np.random.default_rng(topk * 7 + H)
            dout = rng.standard_normal((sub.T, H, sub.d_v)).astype(np.float32)
            fwd = _oracle_forward(sub, sub.idx_main)
            dq, dkv, _, do = run_backward(sub, dout, fwd=fwd)
            check_backward(sub, sub.idx_main, do, dq, dkv, fwd=fwd)
