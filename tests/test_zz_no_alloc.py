"""dsa_decode_static (the fused layer on the library's static scratch, no workspace argument)
against dsa_decode with a caller's workspace: the same kernels, so the results must agree bit
for bit. Calls run back to back on the one static array, each later call on a smaller problem
than the first, so each depends on the previous call having left the control words at zero."""
import pytest
import torch

from dev import dsa, need_gpu, say, upload, workload

pytestmark = [pytest.mark.gpu, need_gpu]


def _buffers(prob):
    T, H = prob.T, prob.H
    return dict(out=torch.full((T, H, prob.d_v), float("nan"), dtype=torch.bfloat16, device="cuda"),
                lse=torch.full((T, H), float("nan"), device="cuda"),
                idx=torch.full((T, prob.topk), -7, dtype=torch.int32, device="cuda"),
                lens=torch.full((T,), -7, dtype=torch.int32, device="cuda"))


def _bits(b):
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu() for k, v in b.items()}


def _run(m, prob, d, static):
    b = _buffers(prob)
    args = (d.q, d.q_idx, d.w, d.keys, d.kv, d.rows, prob.H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
            prob.topk, prob.index_scale, prob.softmax_scale, b["out"], b["lse"], b["idx"], b["lens"])
    if static:
        m.dsa_decode_static(*args)
    else:
        ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_DECODE, T=prob.T, n_max=prob.n_max, topk=prob.topk,
                                              H=prob.H))
        m.dsa_decode(*args, ws)
    torch.cuda.synchronize()
    return _bits(b)


SEQUENCE = [
    ("glm_128k", dict(n_ctx=131072)),                                         # long rows, 64 splits
    ("ragged_20k_b3", dict(n_ctx=20000, B=3, ctx_lens=(20000, 700, 17001))),  # smaller
    ("tiny", dict(n_ctx=512, B=1, H=16, Hi=4, di=64, topk=128, page_size=64)),  # smaller still
]


def test_decode_static_matches_decode_back_to_back():
    m = dsa()
    for label, kw in SEQUENCE:
        prob = workload("glm_decode", **kw)
        d = upload(prob)
        say("decode_static", label)
        got = _run(m, prob, d, static=True)
        ref = _run(m, prob, d, static=False)
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"{label}: {k} differs from dsa_decode"
        assert torch.isfinite(got["lse"]).all()


def test_decode_static_rejects_a_problem_over_the_limit():
    """64 rows of 1M candidates need more scratch than the static array: rejected before any
    launch, and the array stays usable."""
    m = dsa()
    prob = workload("glm_decode", n_ctx=512, B=1, H=16, Hi=4, di=64, topk=128, page_size=64)
    d = upload(prob)
    rows = m.Rows(torch.full((64,), 1 << 20, dtype=torch.int32, device="cuda"), 64, 1 << 20)
    T = 64
    b = dict(out=torch.empty((T, 16, 512), dtype=torch.bfloat16, device="cuda"),
             lse=torch.empty((T, 16), device="cuda"))
    with pytest.raises(m.DSAError) as e:
        m.dsa_decode_static(torch.empty((T, 16, 576), dtype=torch.bfloat16, device="cuda"),
                            torch.empty((T, 4, 64), dtype=torch.bfloat16, device="cuda"),
                            torch.empty((T, 4), device="cuda"), d.keys, d.kv, rows, 16, 576, 512, 4, 64,
                            2048, 1.0, 0.04, b["out"], b["lse"], None, None)
    assert e.value.status == m.DSA_ERR_SCRATCH_LIMIT
    got = _run(m, prob, d, static=True)
    ref = _run(m, prob, d, static=False)
    for k in ref:
        assert torch.equal(got[k], ref[k])
