"""Guard canaries around every output: each output of an entry point lives inside a larger
buffer, with guard elements before and after it and a gap after each row (a row stride larger
than the row), all holding a NaN-like bit pattern before the call. After the call every element
the contract names as written must have changed and every other one must not: no stray or
out-of-bounds write, no write into the caller's row padding, no write of padded heads (H that
is not a whole number of 16-head tiles), no write past the workspace size it was given. A
second layer call on the same workspace gives the same bits (its control words were left as the
next call needs them).

Contracts checked (include/dsa.h): scores write logits[t, 0:n_t] and leave [n_t, ld) alone;
top-k writes indices[t, 0:topk] and lens[t]; attention writes out[t, h, 0:d_v] and lse[t, h]
for h < H; the layer writes all four; the backward writes dq[t, h, 0:d_qk] and adds into dkv.
"""
import ctypes
import dataclasses
import math

import numpy as np
import pytest
import torch

from dev import dsa, need_gpu, say, upload, workload
from workloads.gen import attention_case, grid_base, grid_lists

pytestmark = [pytest.mark.gpu, need_gpu]

G = 4096   # guard elements on each side of an output
_FILL = {torch.bfloat16: (torch.int16, 0x7FA5), torch.float32: (torch.int32, 0x7FC0DEAD),
         torch.int32: (torch.int32, -0x5A5A5A5B), torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """Output [rows, *inner] with row stride ld (elements) inside one flat buffer with G guard
    elements before and after; every element starts as the fill pattern of its dtype."""

    def __init__(self, rows, inner, ld, dtype):
        self.rows, self.cols, self.ld = rows, int(math.prod(inner)), ld
        assert ld >= self.cols
        self.buf = torch.empty(G + rows * ld + G, dtype=dtype, device="cuda")
        itype, self.fill = _FILL[dtype]
        self.bits = self.buf.view(itype)
        self.bits.fill_(self.fill)
        body = self.buf[G:G + rows * ld].view(rows, ld)[:, :self.cols]
        self.t = body.reshape(rows) if not inner else body.view(rows, *inner)

    def check(self, what, written=None):
        """written: per row, the number of leading elements the call must write (all by
        default); the rest of the row, its gap and both guards must still hold the fill."""
        torch.cuda.synchronize()
        b = self.bits.cpu().numpy()
        fill = np.array(self.fill).astype(b.dtype)
        assert (b[:G] == fill).all(), f"{what}: write before the buffer"
        assert (b[G + self.rows * self.ld:] == fill).all(), f"{what}: write past the buffer"
        body = b[G:G + self.rows * self.ld].reshape(self.rows, self.ld)
        wc = np.full(self.rows, self.cols) if written is None else np.asarray(written)
        inside = np.arange(self.ld)[None, :] < wc[:, None]
        bad = np.argwhere(~inside & (body != fill))
        assert bad.size == 0, f"{what}: {len(bad)} stray writes, first at (row, col) {tuple(bad[0])}"
        miss = np.argwhere(inside & (body == fill))
        assert miss.size == 0, f"{what}: {len(miss)} elements not written, first at {tuple(miss[0])}"


class GuardedWorkspace:
    """A workspace of exactly `nbytes` (initialised by the library) followed by a guard."""

    def __init__(self, nbytes):
        m = dsa()
        self.n = int(nbytes)
        self.raw = torch.empty(self.n + G, dtype=torch.uint8, device="cuda")
        self.body = self.raw[:self.n]
        m.dsa_workspace_init(self.body)
        self.raw[self.n:].fill_(0xA5)
        self.ptr = ctypes.c_void_p(self.body.data_ptr())
        self.nbytes = self.n

    def check(self, what):
        torch.cuda.synchronize()
        tail = self.raw[self.n:].cpu().numpy()
        assert (tail == 0xA5).all(), f"{what}: write past the workspace"


def _layer_case(name):
    if name == "short_rows":      # every row in LDS top-k; padded lists (n_t < topk)
        return workload("glm_decode", n_ctx=3000, B=3, ctx_lens=(3000, 1, 777), topk=256, H=40)
    return workload("glm_decode", n_ctx=20000, B=3, ctx_lens=(20000, 700, 17001), H=64)   # long rows


@pytest.mark.parametrize("name", ["short_rows", "long_rows"])
def test_layer_writes_only_its_outputs(name):
    m = dsa()
    prob = _layer_case(name)
    d = upload(prob)
    T, H = prob.T, prob.H
    say(f"guards: dsa_decode {name} T={T} H={H} n_max={prob.n_max} topk={prob.topk}")
    out = Guarded(T, (H, prob.d_v), H * prob.d_v + 40, torch.bfloat16)
    lse = Guarded(T, (H,), H, torch.float32)
    idx = Guarded(T, (prob.topk,), prob.topk + 5, torch.int32)
    lens = Guarded(T, (), 1, torch.int32)
    ws = GuardedWorkspace(m.dsa_workspace_size(m.ENTRY_DECODE, T=T, n_max=prob.n_max, topk=prob.topk, H=H))
    m.dsa_decode(d.q, d.q_idx, d.w, d.keys, d.kv, d.rows, H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
                 prob.topk, prob.index_scale, prob.softmax_scale, out.t, lse.t, idx.t, lens.t, ws)
    out.check("out")
    lse.check("lse")
    idx.check("indices")
    lens.check("lens")
    ws.check("dsa_decode")
    got = lens.t.cpu().numpy()
    assert (got == np.minimum(prob.topk, prob.row_len)).all()
    # the same workspace again: identical results
    out2, lse2 = torch.empty_like(out.t), torch.empty_like(lse.t)
    idx2, lens2 = torch.empty_like(idx.t), torch.empty_like(lens.t)
    m.dsa_decode(d.q, d.q_idx, d.w, d.keys, d.kv, d.rows, H, prob.d_qk, prob.d_v, prob.Hi, prob.di,
                 prob.topk, prob.index_scale, prob.softmax_scale, out2, lse2, idx2, lens2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.t.contiguous().view(torch.int16))
    assert torch.equal(lse2.view(torch.int32), lse.t.view(torch.int32))
    assert torch.equal(idx2, idx.t) and torch.equal(lens2, lens.t)
    ws.check("dsa_decode, second call")


def test_scores_and_topk_write_only_their_outputs():
    m = dsa()
    prob = _layer_case("long_rows")
    d = upload(prob)
    T, k = prob.T, prob.topk
    say(f"guards: dsa_index_scores + dsa_topk T={T} n_max={prob.n_max}")
    logits = Guarded(T, (prob.n_max,), prob.n_max + 3, torch.float32)
    m.dsa_index_scores(d.q_idx, d.w, d.keys, d.rows, prob.Hi, prob.di, prob.index_scale, logits.t)
    logits.check("logits", written=prob.row_len)     # [n_t, ld) stays the caller's
    idx = Guarded(T, (k,), k + 5, torch.int32)
    lens = Guarded(T, (), 1, torch.int32)
    ws = GuardedWorkspace(m.dsa_workspace_size(m.ENTRY_TOPK, T=T, n_max=prob.n_max, topk=k))
    m.dsa_topk(logits.t, d.rows, k, idx.t, lens.t, ws)
    idx.check("indices")
    lens.check("lens")
    ws.check("dsa_topk")


@pytest.mark.parametrize("H", [8, 40])
@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_attention_writes_only_real_heads(mode, H):
    """H = 8 and 40 leave part of a 16-head tile as padding: nothing of it may be written."""
    m = dsa()
    prob = attention_case(fmt="bf16", B=4, H=H, n_ctx=3000, n_idx=700, pad="shuffled", n_pad=50)
    d = upload(prob)
    T = prob.T
    say(f"guards: attention {mode} H={H} T={T}")
    out = Guarded(T, (H, prob.d_v), H * prob.d_v + 24, torch.bfloat16)
    lse = Guarded(T, (H,), H, torch.float32)
    if mode == "decode":
        ws = GuardedWorkspace(m.dsa_workspace_size(m.ENTRY_MLA_DECODE, T=T, H=H, n_idx=int(d.idx_main.shape[1])))
        m.dsa_sparse_mla_decode(d.q, d.kv, d.idx_main, None, None, T, H, prob.d_qk, prob.d_v,
                                prob.softmax_scale, out.t, lse.t, ws)
        ws.check("dsa_sparse_mla_decode")
    else:
        m.dsa_sparse_mla_prefill(d.q, d.kv, d.idx_main, None, None, d.rows, H, prob.d_qk, prob.d_v,
                                 prob.softmax_scale, out.t, lse.t)
    out.check("out")
    lse.check("lse")


@pytest.mark.parametrize("H", [40, 64])
def test_backward_writes_only_dq_and_dkv(H):
    m = dsa()
    base = grid_base("packed", H, seed=5)
    idx = grid_lists(base, 96, "tail", seed=5)
    prob = dataclasses.replace(base, topk=96, idx_main=idx)
    d = upload(prob)
    T = prob.T
    say(f"guards: backward H={H} T={T}")
    out = torch.zeros((T, H, prob.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), device="cuda")
    m.dsa_sparse_mla_prefill(d.q, d.kv, torch.from_numpy(idx).cuda(), None, None, d.rows, H, prob.d_qk,
                             prob.d_v, prob.softmax_scale, out, lse)
    rng = np.random.default_rng(H)
    dout = torch.from_numpy(rng.standard_normal((T, H, prob.d_v)).astype(np.float32)).to(torch.bfloat16).cuda()
    dq = Guarded(T, (H, prob.d_qk), H * prob.d_qk + 16, torch.float32)
    n_slots = int(d.kv.c.n_slots)
    dkv = Guarded(n_slots, (prob.d_qk,), prob.d_qk, torch.float32)
    dkv.t.zero_()                                   # accumulated into: the caller zeroes it
    ws = GuardedWorkspace(m.dsa_workspace_size(m.ENTRY_MLA_BACKWARD, T=T, H=H, n_idx=idx.shape[1]))
    m.dsa_sparse_mla_backward(d.q, d.kv, torch.from_numpy(idx).cuda(), d.rows, H, prob.d_qk, prob.d_v,
                              prob.softmax_scale, out, lse, dout, dq.t, dkv.t, ws)
    dq.check("dq")
    torch.cuda.synchronize()
    b = dkv.bits.cpu().numpy()
    fill = np.array(dkv.fill).astype(b.dtype)
    assert (b[:G] == fill).all() and (b[G + n_slots * prob.d_qk:] == fill).all(), "dkv: write outside"
    assert np.isfinite(dkv.t.cpu().numpy()).all()
    ws.check("dsa_sparse_mla_backward")
