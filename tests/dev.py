"""Shared helpers of the GPU parity tests: cached workloads and one call per entry point."""
import functools

import numpy as np
import pytest
import torch

import workloads as W

GPU = torch.cuda.is_available()
need_gpu = pytest.mark.skipif(not GPU, reason="needs an MI355X")


def say(*a):
    print(*a, flush=True)


@functools.lru_cache(maxsize=4)
def workload(name, **kw):
    kw = dict(kw)
    fn = {"glm_decode": W.glm_decode, "causal_prefill": W.causal_prefill, "tiny_decode": W.tiny_decode,
          "long_decode": W.long_decode, "dsv4_fp8_decode": W.dsv4_fp8_decode,
          "attention_case": W.attention_case}[name]
    if "ctx_lens" in kw and kw["ctx_lens"] is not None:
        kw["ctx_lens"] = list(kw["ctx_lens"])
    if "seg_lens" in kw:
        kw["seg_lens"] = list(kw["seg_lens"])
    return fn(**kw)


def dsa():
    import deepseek_sparse_attention_indexer_amd as m
    return m


def upload(prob):
    from deepseek_sparse_attention_indexer_amd.upload import to_device
    return to_device(prob, "cuda")


def run_scores(prob, d=None, ld_pad=3):
    m = dsa()
    d = d or upload(prob)
    ld = prob.n_max + ld_pad
    logits = torch.full((prob.T, ld), float("nan"), device="cuda")
    m.dsa_index_scores(d.q_idx, d.w, d.keys, d.rows, prob.Hi, prob.di, prob.index_scale, logits)
    torch.cuda.synchronize()
    return logits


def run_topk(logits, row_len, n_req, k, ws=None, ld_idx=None):
    m = dsa()
    T = logits.shape[0]
    rl = torch.as_tensor(np.asarray(row_len, np.int32)).cuda()
    rows = m.Rows(rl, n_req, int(np.max(row_len)) if T else 0)
    ld_idx = ld_idx or k
    idx = torch.full((T, ld_idx), -7, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_TOPK, T=T, n_max=rows.c.n_max, topk=k))
    m.dsa_topk(logits, rows, k, idx, lens, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), lens.cpu().numpy()


def run_attention(prob, d=None, mode="decode", idx=None):
    """mode 'decode' (split-KV entry) or 'prefill' (one workgroup per row)."""
    m = dsa()
    d = d or upload(prob)
    idx_main = d.idx_main if idx is None else idx
    out = torch.full((prob.T, prob.H, prob.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((prob.T, prob.H), float("nan"), device="cuda")
    n_idx = int(idx_main.shape[1]) + (int(d.idx_extra.shape[1]) if d.idx_extra is not None else 0)
    if mode == "decode":
        ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_MLA_DECODE, T=prob.T, H=prob.H, n_idx=n_idx))
        m.dsa_sparse_mla_decode(d.q, d.kv, idx_main, d.extra_kv, d.idx_extra, prob.T, prob.H, prob.d_qk,
                                prob.d_v, prob.softmax_scale, out, lse, ws, sink=d.sink, lse_log2=d.lse_log2)
    else:
        m.dsa_sparse_mla_prefill(d.q, d.kv, idx_main, d.extra_kv, d.idx_extra, d.rows, prob.H, prob.d_qk,
                                 prob.d_v, prob.softmax_scale, out, lse, sink=d.sink, lse_log2=d.lse_log2)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def run_decode(prob, d=None):
    m = dsa()
    d = d or upload(prob)
    T, H = prob.T, prob.H
    out = torch.full((T, H, prob.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), device="cuda")
    idx = torch.full((T, prob.topk), -7, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_DECODE, T=T, n_max=prob.n_max, topk=prob.topk, H=H))
    m.dsa_decode(d.q, d.q_idx, d.w, d.keys, d.kv, d.rows, H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
                 prob.topk, prob.index_scale, prob.softmax_scale, out, lse, idx, lens, ws,
                 sink=d.sink, lse_log2=d.lse_log2)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), lens.cpu().numpy()


def bf16_round(x):
    """float array -> the float64 values of its bf16 rounding (RNE, torch cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy() \
        .astype(np.float64)


def run_backward(prob, dout, d=None, idx=None, with_dsink=False, fwd=None, owner=True, ws=None):
    """The backward. Its forward outputs: fwd = (out [T, H, d_v], lse [T, H]) given as numpy
    (out is rounded to bf16, lse to fp32 on the way in), or None for the GPU's own forward
    (one workgroup per row). dout: float32 numpy [T, H, d_v], rounded to bf16 here (the tests
    hand the same bf16 values to the oracle).
    owner: size the workspace with the cache's slot count (the owner map: plain adds for slots
    one entry alone names), else without (every dKV add atomic). ws: a workspace to use instead.
    Returns (dq [T, H, d_qk], dkv [n_slots, d_qk], dsink [H] or None, dout as float64)."""
    m = dsa()
    d = d or upload(prob)
    idx_main = d.idx_main if idx is None else idx
    T, H = prob.T, prob.H
    if fwd is None:
        out = torch.full((T, H, prob.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), float("nan"), device="cuda")
        m.dsa_sparse_mla_prefill(d.q, d.kv, idx_main, None, None, d.rows, H, prob.d_qk, prob.d_v,
                                 prob.softmax_scale, out, lse, sink=d.sink, lse_log2=d.lse_log2)
    else:
        out = torch.from_numpy(np.ascontiguousarray(fwd[0], dtype=np.float32)).to(torch.bfloat16).cuda()
        lse = torch.from_numpy(np.ascontiguousarray(fwd[1], dtype=np.float32)).cuda()
    do = torch.from_numpy(np.ascontiguousarray(dout, dtype=np.float32)).to(torch.bfloat16).cuda()
    dq = torch.full((T, H, prob.d_qk), float("nan"), device="cuda")
    dkv = torch.zeros((int(d.kv.c.n_slots), prob.d_qk), device="cuda")
    dsink = torch.zeros((H,), device="cuda") if with_dsink else None
    if ws is None:
        ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_MLA_BACKWARD, T=T, H=H, n_idx=int(idx_main.shape[1]),
                                              n_slots=int(d.kv.c.n_slots) if owner else 0))
    m.dsa_sparse_mla_backward(d.q, d.kv, idx_main, d.rows, H, prob.d_qk, prob.d_v, prob.softmax_scale,
                              out, lse, do, dq, dkv, ws, dsink, sink=d.sink, lse_log2=d.lse_log2)
    torch.cuda.synchronize()
    return (dq.cpu().numpy(), dkv.cpu().numpy(), dsink.cpu().numpy() if with_dsink else None,
            do.float().cpu().numpy().astype(np.float64))
