"""Backward of the sparse attention on the GPU (dsa_sparse_mla_backward) against the fp64
oracle's exact gradient (step 5 of the oracle's description).

The kernel's inputs are bf16 and exact; what it rounds: P and scale * dZ to bf16 as MFMA
operands (2^-9 relative per term), fp32 accumulation (and fp32 atomics in any order for dkv).
dq and dkv are held to 2% of the largest reference value of the (row, head) and of the whole
dkv respectively (measured worst: 0.3% and 0.4%).

Two ways to feed the backward its forward outputs (out, lse):
* the oracle's forward, out rounded to bf16 and lse to fp32 (test_backward): the reference is
  the oracle's gradient taken at those same given outputs (D from the given out, P from the
  given lse), so no forward error is charged to the backward, and the sink gradient, which
  needs no bf16 operand, is held to 2e-2 relative;
* the GPU's own forward (test_backward_chained, the end-to-end case): the reference is the
  exact gradient, and the sink gradient is held to a bound derived from the rounding of D
  that the bf16 out brings (below)."""
import numpy as np
import pytest

import oracle
from dev import bf16_round, need_gpu, run_backward, say, upload, workload

pytestmark = [pytest.mark.gpu, need_gpu]

CASES = [
    ("bf16_576_tail", dict(fmt="bf16", B=3, H=16, n_ctx=700, n_idx=96, pad="tail", n_pad=10)),
    ("bf16_576_h64_two_passes", dict(fmt="bf16", B=2, H=64, n_ctx=3000, n_idx=2048, pad="shuffled", n_pad=100)),
    ("bf16_512", dict(fmt="bf16", B=2, H=32, n_ctx=500, n_idx=70, d_nope=448, d_v=512, n_pad=0)),
    ("bf16_sink_log2", dict(fmt="bf16", B=3, H=16, n_ctx=700, n_idx=96, pad="tail", n_pad=10,
                            sink=True, lse_log2=True)),
    ("bf16_all_padded", dict(fmt="bf16", B=2, H=16, n_ctx=300, n_idx=64, pad="all")),
    # head counts padded inside: 8 (one 16-head group) and 40 (64 in the dKV head sum)
    ("bf16_576_h8_sink", dict(fmt="bf16", B=3, H=8, n_ctx=700, n_idx=96, pad="tail", n_pad=10, sink=True)),
    ("bf16_576_h40", dict(fmt="bf16", B=2, H=40, n_ctx=900, n_idx=300, pad="shuffled", n_pad=20)),
    # a row's list in four parts (two rows fill too few workgroups) of 1280 entries: two
    # resolve passes of 1024 each, and the parts' dq partial sums added afterwards
    ("bf16_576_h64_parts_two_passes", dict(fmt="bf16", B=2, H=64, n_ctx=6000, n_idx=5000, pad="shuffled", n_pad=200)),
]


def _reference(prob, idx, dout, fwd=None):
    T, H = prob.T, prob.H
    dq = np.zeros((T, H, prob.d_qk))
    dkv = {}
    dsink = np.zeros(H)
    for t in range(T):
        given = {} if fwd is None else {"out": fwd[0][t], "lse": fwd[1][t]}
        q_t, slots, drows, ds = oracle.attention_backward_row(prob, t, idx[t], dout[t], **given)
        dq[t] = q_t
        for s, r in zip(slots.tolist(), drows[:, :prob.d_qk]):
            dkv[s] = dkv.get(s, 0.0) + r
        dsink += ds
    return dq, dkv, dsink


def _check(prob, idx, dout, dq, dkv, dsink=None, fwd=None):
    """fwd: the (out, lse) the kernel was handed, as the float64 values it received, or None
    (the GPU's own forward; the reference is then the exact gradient)."""
    dq_ref, dkv_ref, dsink_ref = _reference(prob, idx, dout, fwd)
    err = np.abs(dq - dq_ref)
    scale = np.abs(dq_ref).max(axis=2, keepdims=True)
    worst = float((err / (scale + 1e-30)).max()) if dq_ref.size else 0.0
    say("  dq: max err", float(err.max()), "worst relative to the (row, head) max", worst)
    assert np.all(err <= 2e-2 * scale + 1e-5), "dq"
    touched = np.zeros(dkv.shape[0], bool)
    if dkv_ref:
        slots = np.array(sorted(dkv_ref))
        ref = np.stack([dkv_ref[s] for s in slots])
        got = dkv[slots]
        touched[slots] = True
        e = np.abs(got - ref)
        say("  dkv: max err", float(e.max()), "max |ref|", float(np.abs(ref).max()),
            "frobenius rel", float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
        assert np.all(e <= 2e-2 * np.abs(ref).max() + 1e-5), "dkv"
    assert np.all(dkv[~touched] == 0.0), "dkv rows outside the lists changed"
    if dsink is not None and fwd is not None:
        # the reference takes D from the same bf16 out and p_sink from the same lse: what is
        # left is fp32 arithmetic (and atomic order), far inside 2e-2 relative; the floor covers
        # a head whose rows' terms cancel
        terms = np.zeros(prob.H)
        sink = np.asarray(prob.sink, dtype=np.float64)
        base = np.log(2.0) if getattr(prob, "lse_log2", False) else 1.0
        for t in range(prob.T):
            terms += np.exp(sink - fwd[1][t] * base) * np.abs((dout[t] * fwd[0][t]).sum(axis=1))
        err = np.abs(dsink - dsink_ref)
        say("  dsink: max err", float(err.max()), "max rel", float((err / (np.abs(dsink_ref) + 1e-30)).max()))
        assert np.all(err <= 2e-2 * np.abs(dsink_ref) + 1e-6 * terms + 1e-7), "dsink"
    elif dsink is not None:
        # dsink_h = -sum_t p_sink D with D = dout . out, and the kernel takes D from the forward's
        # bf16 out (rounding error <= 2^-9 per element): |error| <= sum_t p_sink 2^-8 sum_d
        # |dout| |out| (a factor 2 for the fp32 sum), which stays the same when D cancels
        bound = np.zeros(prob.H)
        sink = np.asarray(prob.sink, dtype=np.float64)
        base = np.log(2.0) if getattr(prob, "lse_log2", False) else 1.0
        for t in range(prob.T):
            out_ref, lse_ref = oracle.attention_row(prob, t, idx[t])
            p_sink = np.exp(sink - lse_ref * base)
            bound += p_sink * 2.0 ** -8 * (np.abs(dout[t]) * np.abs(out_ref)).sum(axis=1)
        say("  dsink: max err", float(np.abs(dsink - dsink_ref).max()), "bound", float(bound.max()))
        assert np.all(np.abs(dsink - dsink_ref) <= bound + 2.0 ** -8 * np.abs(dsink_ref) + 1e-5), "dsink"


def _oracle_forward(prob, idx):
    """The oracle's forward outputs as the backward receives them: out rounded to bf16 (RNE),
    lse to fp32, both returned as the float64 values handed over."""
    outs, lses = [], []
    for t in range(prob.T):
        o, l = oracle.attention_row(prob, t, idx[t])
        outs.append(o)
        lses.append(l)
    out = bf16_round(np.stack(outs))
    lse = np.stack(lses).astype(np.float32).astype(np.float64)
    return out, lse


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_backward(name, kw):
    """The backward on the oracle's forward outputs."""
    prob = workload("attention_case", **kw)
    say("backward (oracle forward)", name)
    rng = np.random.default_rng(len(name))
    dout = rng.standard_normal((prob.T, prob.H, prob.d_v)).astype(np.float32)
    with_dsink = getattr(prob, "sink", None) is not None
    fwd = _oracle_forward(prob, prob.idx_main)
    dq, dkv, dsink, do = run_backward(prob, dout, with_dsink=with_dsink, fwd=fwd)
    _check(prob, prob.idx_main, do, dq, dkv, dsink, fwd=fwd)


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_backward_chained(name, kw):
    """End to end: the GPU's forward, then the backward, against the exact gradient."""
    prob = workload("attention_case", **kw)
    say("backward (GPU forward)", name)
    rng = np.random.default_rng(len(name))
    dout = rng.standard_normal((prob.T, prob.H, prob.d_v)).astype(np.float32)
    with_dsink = getattr(prob, "sink", None) is not None
    dq, dkv, dsink, do = run_backward(prob, dout, with_dsink=with_dsink)
    _check(prob, prob.idx_main, do, dq, dkv, dsink)


@pytest.mark.parametrize("name,kw", [c for c in CASES if c[1]["H"] > 16], ids=[c[0] for c in CASES if c[1]["H"] > 16])
def test_backward_atomics_only(name, kw):
    """The dKV kernel without the owner map (a workspace sized without n_slots): every add
    atomic, same results."""
    prob = workload("attention_case", **kw)
    say("backward (atomics only)", name)
    rng = np.random.default_rng(len(name))
    dout = rng.standard_normal((prob.T, prob.H, prob.d_v)).astype(np.float32)
    with_dsink = getattr(prob, "sink", None) is not None
    fwd = _oracle_forward(prob, prob.idx_main)
    dq, dkv, dsink, do = run_backward(prob, dout, with_dsink=with_dsink, fwd=fwd, owner=False)
    _check(prob, prob.idx_main, do, dq, dkv, dsink, fwd=fwd)


@pytest.mark.parametrize("H", [16, 64])
def test_backward_repeated_entry(H):
    """An entry listed twice contributes twice (to the softmax and to dKV). With 64 heads the
    owner map must see the slot named twice and keep its adds atomic."""
    import torch
    prob = workload("attention_case", fmt="bf16", B=2, H=H, n_ctx=400, n_idx=40, n_pad=0)
    idx = prob.idx_main.copy()
    idx[:, 5] = idx[:, 3]
    say("backward repeated entry, H", H)
    d = upload(prob)
    rng = np.random.default_rng(3)
    dout = rng.standard_normal((prob.T, prob.H, prob.d_v)).astype(np.float32)
    dq, dkv, _, do = run_backward(prob, dout, d=d, idx=torch.from_numpy(idx).cuda())
    _check(prob, idx, do, dq, dkv)


def test_backward_rows_sharing_a_request():
    """Four rows of one request with overlapping lists (128 of 300 positions each): slots named
    by several rows take atomics, the others plain adds; both against the oracle."""
    import dataclasses
    base = workload("attention_case", fmt="bf16", B=4, H=64, n_ctx=300, n_idx=128, pad="shuffled", n_pad=8)
    prob = dataclasses.replace(base, row_req=np.zeros(4, dtype=np.int32))
    say("backward, 4 rows of one request")
    slots_named = {}
    for t in range(prob.T):
        for p in prob.idx_main[t]:
            if p >= 0:
                slots_named[int(p)] = slots_named.get(int(p), 0) + 1
    assert 0 < sum(v == 1 for v in slots_named.values()) < len(slots_named)   # both kinds occur
    rng = np.random.default_rng(11)
    dout = rng.standard_normal((prob.T, prob.H, prob.d_v)).astype(np.float32)
    fwd = _oracle_forward(prob, prob.idx_main)
    dq, dkv, _, do = run_backward(prob, dout, fwd=fwd)
    _check(prob, prob.idx_main, do, dq, dkv, fwd=fwd)


def test_backward_owner_map_dirty_then_reused():
    """The owner map may start dirty (a workspace that held other data, or one whose layout
    moved): such words only send their rows to atomics. The dKV kernel clears the words it
    reads, so a second call on the same workspace gets plain adds again. Both calls against
    the oracle."""
    import torch
    from dev import dsa
    m = dsa()
    prob = workload("attention_case", fmt="bf16", B=3, H=64, n_ctx=600, n_idx=256, pad="shuffled", n_pad=16)
    d = upload(prob)
    n_slots = int(d.kv.c.n_slots)
    start = m.dsa_workspace_size(m.ENTRY_MLA_BACKWARD, T=prob.T, H=prob.H, n_idx=256)
    end = m.dsa_workspace_size(m.ENTRY_MLA_BACKWARD, T=prob.T, H=prob.H, n_idx=256, n_slots=n_slots)
    ws = m.Workspace(end)
    g = torch.Generator(device="cpu").manual_seed(5)
    ws.buf[start:end].copy_(torch.randint(0, 256, (end - start,), generator=g, dtype=torch.uint8))
    rng = np.random.default_rng(21)
    dout = rng.standard_normal((prob.T, prob.H, prob.d_v)).astype(np.float32)
    fwd = _oracle_forward(prob, prob.idx_main)
    for call in range(2):
        say("backward on a dirty owner map, call", call)
        dq, dkv, _, do = run_backward(prob, dout, d=d, fwd=fwd, ws=ws)
        _check(prob, prob.idx_main, do, dq, dkv, fwd=fwd)
        if call == 0:   # every listed slot's word is back to 0
            words = ws.buf[start:end].view(torch.int32).cpu().numpy()
            slots = set()
            for t in range(prob.T):
                for p in prob.idx_main[t]:
                    if p >= 0:
                        slots.add(int(prob.kv.block_table[t, p // prob.kv.page_size]) * prob.kv.page_size
                                  + int(p) % prob.kv.page_size)
            assert all(words[s] == 0 for s in slots)


def test_backward_full_size_sampled_rows():
    """The measured backward shape at full size: 64 rows (each its own request) x 64 heads x
    2048 listed of 4096 cached rows, the GPU's forward then the backward with the owner map
    (every listed cache row is named once: whole-row plain adds). dq and the dKV rows of five
    sampled query rows against the exact gradient; each dKV row holds one entry's
    contribution, so a row's slots compare on their own."""
    prob = workload("attention_case", fmt="bf16", B=64, H=64, n_ctx=4096, n_idx=2048, pad="tail", n_pad=0)
    say("backward full size, 64 x 64 x 2048")
    rng = np.random.default_rng(64)
    dout = rng.standard_normal((prob.T, prob.H, prob.d_v)).astype(np.float32)
    dq, dkv, _, do = run_backward(prob, dout)
    for t in (0, 1, 17, 40, 63):
        dq_ref, slots, drows, _ = oracle.attention_backward_row(prob, t, prob.idx_main[t], do[t])
        scale = np.abs(dq_ref).max(axis=1, keepdims=True)
        err = np.abs(dq[t] - dq_ref)
        ref = drows[:, :prob.d_qk]
        e = np.abs(dkv[slots] - ref)
        say("  row", t, "dq worst rel", float((err / (scale + 1e-30)).max()),
            "dkv max err", float(e.max()), "max |ref|", float(np.abs(ref).max()))
        assert np.all(err <= 2e-2 * scale + 1e-5), f"dq row {t}"
        assert np.all(e <= 2e-2 * np.abs(ref).max() + 1e-5), f"dkv rows of row {t}"
