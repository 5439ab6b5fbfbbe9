"""Indexer scores on the GPU (dsa_index_scores) against the fp64 oracle, element by element."""
import numpy as np
import pytest

import oracle
from oracle.compare import scores_ok
from dev import need_gpu, run_scores, say, workload

pytestmark = [pytest.mark.gpu, need_gpu]

SMALL = [
    ("tiny_decode", dict()),
    ("glm_decode", dict(n_ctx=3000, B=3, ctx_lens=(3000, 1, 777), make_kv=False)),
    ("glm_decode", dict(n_ctx=2500, B=2, ctx_lens=(2500, 1999), key_dtype="fp8", make_kv=False)),
    ("glm_decode", dict(n_ctx=1000, Hi=20, di=64, w_low=-1.0, index_scale=0.125, make_kv=False)),
    ("glm_decode", dict(n_ctx=1000, Hi=32, page_size=16, make_kv=False)),
    ("glm_decode", dict(n_ctx=777, Hi=64, page_size=48, make_kv=False)),
    ("glm_decode", dict(n_ctx=640, Hi=16, di=64, key_dtype="fp8", make_kv=False)),
    ("causal_prefill", dict(seg_lens=(300, 1, 45))),
    # 10 requests x 8 query tokens (80 rows > requests: the shared-key prefill kernel) on a
    # paged cache with 48-token pages, rows crossing the 8192-position chunk boundary
    ("glm_decode", dict(n_ctx=9000, B=10, q_len=8, page_size=48, make_kv=False,
                        ctx_lens=(9000, 8, 8200, 100, 8193, 4097, 50, 8999, 2000, 9))),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_scores_small(name, kw):
    prob = workload(name, **kw)
    say("scores", prob.name, prob.T, prob.n_max)
    logits = run_scores(prob).cpu().numpy()
    for t in range(prob.T):
        n = int(prob.row_len[t])
        ok, msg = scores_ok(logits[t, :n], oracle.index_scores_row(prob, t))
        assert ok, f"row {t}: {msg}"
        assert np.all(np.isnan(logits[t, n:])), "wrote past the row's candidates"


@pytest.mark.parametrize("n_ctx,key_dtype", [(32768, "bf16"), (131072, "bf16"), (1 << 20, "fp8")])
def test_scores_full_size_decode(n_ctx, key_dtype):
    """The GLM decode shapes (32k, 128k) and the 1M fp8-key shape: every score of the row at
    128k and below; at 1M a seeded sample of 65536 positions plus the ragged end."""
    prob = workload("glm_decode", n_ctx=n_ctx, key_dtype=key_dtype, make_kv=False)
    say("scores full", n_ctx, key_dtype)
    logits = run_scores(prob).cpu().numpy()[0]
    if n_ctx <= 131072:
        pos = np.arange(n_ctx)
    else:
        pos = np.unique(np.concatenate([np.random.default_rng(1).choice(n_ctx, 65536, replace=False),
                                        np.arange(n_ctx - 100, n_ctx)]))
    ref = oracle.index_scores_row(prob, 0, pos)
    full_max = np.abs(ref).max()
    ok, msg = scores_ok(logits[pos], ref)
    assert ok, msg
    assert np.isfinite(logits[:n_ctx]).all() and full_max > 0


def test_scores_full_size_causal_prefill_sampled_rows():
    """Causal prefill of one 8192-token segment plus a 1-token segment: whole score rows at
    sampled query positions (first, around topk, last of each segment)."""
    prob = workload("causal_prefill", seg_lens=(8192, 1))
    say("scores prefill 8193 rows")
    logits = run_scores(prob).cpu().numpy()
    for t in [0, 1, 63, 64, 2046, 2047, 2048, 4097, 8191, 8192]:
        n = int(prob.row_len[t])
        ok, msg = scores_ok(logits[t, :n], oracle.index_scores_row(prob, t))
        assert ok, f"row {t}: {msg}"


def test_scores_fp8_keys_with_negative_scales():
    """fp8 keys whose per-token scale is negative for some tokens (the cache writer never makes
    one, but the formula takes any scale): every score still matches the oracle."""
    import dataclasses
    base = workload("glm_decode", n_ctx=3000, B=2, ctx_lens=(3000, 1999), key_dtype="fp8", make_kv=False)
    scale = base.kpool.scale.copy()
    scale[::3] *= -1.0
    scale[5::7] = 0.0
    prob = dataclasses.replace(base, kpool=dataclasses.replace(base.kpool, scale=scale))
    say("scores fp8 negative scales")
    logits = run_scores(prob).cpu().numpy()
    for t in range(prob.T):
        n = int(prob.row_len[t])
        ok, msg = scores_ok(logits[t, :n], oracle.index_scores_row(prob, t))
        assert ok, f"row {t}: {msg}"
