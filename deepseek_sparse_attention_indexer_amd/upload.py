"""Move a problem description (host numpy arrays) into device tensors and ABI descriptors.

Marshalling only: copies bytes and wraps them in KeyCache / KVCache / Rows. Any object with
the attribute names below works (duck typing).
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch

from ._binding import KeyCache, KVCache, Rows


def _t(a, device, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def _kv(pool, device) -> KVCache:
    if pool.fmt == "bf16":
        data = _t(pool.data.view(np.int16), device, torch.bfloat16)
    else:
        data = _t(pool.data, device)
    return KVCache(pool.fmt, data, pool.d_nope, pool.d_rope, page_size=pool.page_size,
                   block_table=_t(pool.block_table, device), req_base=_t(pool.req_base, device),
                   scales=_t(pool.scales, device))


def to_device(prob, device="cuda") -> SimpleNamespace:
    d = SimpleNamespace()
    d.q = _t(prob.q.view(np.int16), device, torch.bfloat16) if prob.q is not None else None
    d.kv = _kv(prob.kv, device) if prob.kv is not None else None
    d.extra_kv = _kv(prob.extra_kv, device) if prob.extra_kv is not None else None
    d.row_len = _t(prob.row_len.astype(np.int32), device)
    d.row_req = _t(prob.row_req.astype(np.int32), device)
    d.rows = Rows(d.row_len, prob.n_req, prob.n_max, row_req=d.row_req)
    if prob.kpool is not None:
        kp = prob.kpool
        kdata = _t(kp.data.view(np.int16), device, torch.bfloat16) if kp.dtype == "bf16" else _t(kp.data, device)
        d.keys = KeyCache(kdata, scale=_t(kp.scale, device), page_size=kp.page_size,
                          block_table=_t(kp.block_table, device), req_base=_t(kp.req_base, device))
        d.q_idx = _t(prob.q_idx.view(np.int16), device, torch.bfloat16)
        d.w = _t(prob.w, device)
    d.idx_main = _t(prob.idx_main, device) if prob.idx_main is not None else None
    d.idx_extra = _t(prob.idx_extra, device) if prob.idx_extra is not None else None
    sink = getattr(prob, "sink", None)
    d.sink = _t(np.asarray(sink, dtype=np.float32), device) if sink is not None else None
    d.lse_log2 = bool(getattr(prob, "lse_log2", False))
    return d
