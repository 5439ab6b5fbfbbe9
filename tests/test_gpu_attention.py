"""Sparse MLA attention on the GPU (decode and prefill entries) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from oracle.compare import attention_ok
from dev import need_gpu, run_attention, say, upload, workload

pytestmark = [pytest.mark.gpu, need_gpu]

CASES = [
    ("bf16_tail", dict(fmt="bf16", B=3, H=16, n_ctx=700, n_idx=96, pad="tail", n_pad=10)),
    ("bf16_shuffled_h64_split", dict(fmt="bf16", B=2, H=64, n_ctx=3000, n_idx=2048, pad="shuffled", n_pad=100)),
    ("bf16_all_padded", dict(fmt="bf16", B=2, H=16, n_ctx=300, n_idx=64, pad="all")),
    # block counts equal to the number of row streams + 1 (a stale-buffer hazard on the pages)
    ("bf16_h16_k128", dict(fmt="bf16", B=1, H=16, n_ctx=1000, n_idx=128, n_pad=0)),
    ("bf16_h16_k160", dict(fmt="bf16", B=1, H=16, n_ctx=1000, n_idx=160, n_pad=0)),
    ("bf16_h16_k192", dict(fmt="bf16", B=1, H=16, n_ctx=1000, n_idx=192, n_pad=0)),
    ("bf16_h32_odd", dict(fmt="bf16", B=3, H=32, n_ctx=900, n_idx=333, pad="shuffled", n_pad=7)),
    ("bf16_h128", dict(fmt="bf16", B=1, H=128, n_ctx=600, n_idx=300, pad="tail", n_pad=3)),
    ("bf16_d512", dict(fmt="bf16", B=2, H=16, n_ctx=500, n_idx=70, d_nope=448, d_v=512, n_pad=0)),
    ("uniform_512", dict(fmt="fp8_uniform", B=2, H=16, n_ctx=800, n_idx=200, pad="shuffled", n_pad=9)),
    ("uniform_576", dict(fmt="fp8_uniform", B=2, H=16, n_ctx=800, n_idx=100, d_nope=512, d_v=512)),
    ("ds_mla_one_list", dict(fmt="fp8_ds_mla", B=2, H=16, n_ctx=2000, n_idx=300, page_size=256,
                             pad="shuffled", n_pad=20)),
    ("ds_mla_two_lists", dict(fmt="fp8_ds_mla", B=3, H=16, n_ctx=2000, n_idx=128, page_size=256,
                              n_extra=300, pad="tail", n_pad=5)),
    ("ds_mla_h64_two_lists", dict(fmt="fp8_ds_mla", B=2, H=64, n_ctx=5000, n_idx=128, page_size=256,
                                  n_extra=1024, pad="shuffled", n_pad=30)),
]


def _check_all(prob, out, lse, rows=None):
    fmt = prob.kv.fmt
    for t in (range(prob.T) if rows is None else rows):
        o_ref, l_ref = oracle.attention_row(prob, t, prob.idx_main[t],
                                            prob.idx_extra[t] if prob.idx_extra is not None else None)
        ok, msg = attention_ok(out[t], lse[t], o_ref, l_ref, fmt)
        assert ok, f"row {t}: {msg}"


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_attention(name, kw, mode):
    prob = workload("attention_case", **kw)
    say("attention", name, mode)
    out, lse = run_attention(prob, mode=mode)
    _check_all(prob, out, lse)


def test_attention_dsv4_fp8_full_size():
    """DeepSeek-V4-style fp8 paged decode at full size: 64 requests, 16 heads, 128 window rows
    in the main cache + 1024 top-k rows in the compressed cache, packed fp8_ds_mla pages."""
    prob = workload("dsv4_fp8_decode")
    say("attention dsv4 full")
    out, lse = run_attention(prob, mode="decode")
    _check_all(prob, out, lse)
