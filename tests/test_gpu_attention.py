"""Sparse MLA attention on the GPU (decode and prefill entries) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from oracle.compare import attention_ok
from workloads.gen import to_bf16_bits
from dev import dsa, need_gpu, run_attention, say, upload, workload

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
    # DeepSeek-V4 options: fnuz uniform pools, attention sinks, base-2 lse
    ("fnuz_512", dict(fmt="fp8_uniform_fnuz", B=2, H=16, n_ctx=800, n_idx=200, pad="shuffled", n_pad=9)),
    ("fnuz_576_two_lists", dict(fmt="fp8_uniform_fnuz", B=2, H=32, n_ctx=900, n_idx=64, n_extra=150,
                                d_nope=512, d_v=512, n_pad=4)),
    ("bf16_sink_log2", dict(fmt="bf16", B=3, H=16, n_ctx=700, n_idx=96, pad="tail", n_pad=10,
                            sink=True, lse_log2=True)),
    ("bf16_sink_h64_split", dict(fmt="bf16", B=2, H=64, n_ctx=3000, n_idx=2048, pad="shuffled",
                                 n_pad=100, sink=True)),
    ("bf16_all_padded_sink", dict(fmt="bf16", B=2, H=16, n_ctx=300, n_idx=64, pad="all", sink=True,
                                  lse_log2=True)),
    # 16 rows x 64 heads in decode: 8-wave 64-head workgroups (each wave finishes 8 rows of
    # the softmax) with splits (ragged last block, padding spread over the lists), for every
    # row format and width, with sinks and a base-2 lse
    ("bf16_h64_b16_ring", dict(fmt="bf16", B=16, H=64, n_ctx=5000, n_idx=2000, pad="shuffled", n_pad=77)),
    ("ds_mla_h64_b16_ring_two_lists", dict(fmt="fp8_ds_mla", B=16, H=64, n_ctx=5000, n_idx=1000,
                                           page_size=64, n_extra=230, pad="tail", n_pad=7)),
    ("uniform_h64_b16", dict(fmt="fp8_uniform", B=16, H=64, n_ctx=3000, n_idx=700, pad="shuffled",
                             n_pad=11)),
    ("fnuz_576_h64_b16_two_lists", dict(fmt="fp8_uniform_fnuz", B=16, H=64, n_ctx=1500, n_idx=256,
                                        n_extra=100, d_nope=512, d_v=512, n_pad=3)),
    ("bf16_d512_h64_b16_sink_log2", dict(fmt="bf16", B=16, H=64, n_ctx=2000, n_idx=600, d_nope=448,
                                         d_v=512, pad="shuffled", n_pad=5, sink=True, lse_log2=True)),
    ("ds_mla_two_lists_sink_log2", dict(fmt="fp8_ds_mla", B=3, H=16, n_ctx=2000, n_idx=128,
                                        page_size=256, n_extra=300, pad="tail", n_pad=5, sink=True,
                                        lse_log2=True)),
    # head counts that are not whole 16-head tiles (the missing heads of the last tile are
    # padding): 8 heads (the TP=8 share of 64), 40, and 56 on the 64-head workgroups
    ("bf16_h8_split", dict(fmt="bf16", B=2, H=8, n_ctx=3000, n_idx=2048, pad="shuffled", n_pad=100)),
    ("ds_mla_h8_two_lists_sink", dict(fmt="fp8_ds_mla", B=3, H=8, n_ctx=2000, n_idx=128, page_size=256,
                                      n_extra=300, pad="tail", n_pad=5, sink=True)),
    ("bf16_h40", dict(fmt="bf16", B=3, H=40, n_ctx=900, n_idx=333, pad="shuffled", n_pad=7, sink=True)),
    ("bf16_h56_b16", dict(fmt="bf16", B=16, H=56, n_ctx=2000, n_idx=600, pad="shuffled", n_pad=5,
                          sink=True, lse_log2=True)),
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


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_sink_edge_values(mode):
    """Per-head sinks at the ends of the range: -inf (no sink for that head), far above every
    logit (out -> 0, lse -> sink), and far below; the others ordinary."""
    import dataclasses
    base = workload("attention_case", fmt="bf16", B=2, H=16, n_ctx=700, n_idx=256, pad="shuffled",
                    n_pad=20, sink=True)
    sink = base.sink.copy()
    sink[0], sink[1], sink[2], sink[3] = -np.inf, 80.0, -80.0, 0.0
    for log2 in (False, True):
        prob = dataclasses.replace(base, sink=sink, lse_log2=log2)
        say("attention sink edges", mode, "log2" if log2 else "ln")
        out, lse = run_attention(prob, mode=mode)
        _check_all(prob, out, lse)


def _fnuz_case(codes, scale):
    import dataclasses
    base = workload("attention_case", fmt="fp8_uniform_fnuz", B=2, H=16, n_ctx=500, n_idx=128,
                    pad="shuffled", n_pad=8)
    rng = np.random.default_rng(len(codes))
    data = rng.choice(np.asarray(codes, np.uint8), size=base.kv.data.shape)
    kv = dataclasses.replace(base.kv, data=data, scales=np.full_like(base.kv.scales, scale))
    return dataclasses.replace(base, kv=kv)


@pytest.mark.parametrize("which", ["subnormal", "ends"])
def test_fnuz_extreme_codes(which):
    """Every fnuz byte class decodes exactly: subnormal codes (m / 8 * 2^-7, decoded through fp32
    denormals) scaled up to unit size, and +-240 (0x7F / 0xFF, NaN codes in OCP) beside zero."""
    if which == "subnormal":
        codes = [c | s for c in range(1, 8) for s in (0, 0x80)]
        prob = _fnuz_case(codes, 256.0)
    else:
        codes = [0x7F, 0xFF, 0x00, 0x38, 0xB8]
        prob = _fnuz_case(codes, 1.0 / 128)
    say("attention fnuz codes", which)
    out, lse = run_attention(prob, mode="decode")
    _check_all(prob, out, lse)
    assert np.abs(out).max() > 0.05        # the rows are not (wrongly) all zero


def test_attention_dsv4_fp8_full_size():
    """DeepSeek-V4-style fp8 paged decode at full size: 64 requests, 16 heads, 128 window rows
    in the main cache + 1024 top-k rows in the compressed cache, packed fp8_ds_mla pages."""
    prob = workload("dsv4_fp8_decode")
    say("attention dsv4 full")
    out, lse = run_attention(prob, mode="decode")
    _check_all(prob, out, lse)


# forced launch plans (dsa_launch_override): every head-tile layout and split count the table
# would not pick for this shape gives the same results
@pytest.mark.parametrize("ht,split", [(1, 1), (1, 7), (2, 3), (4, 1), (4, 5), (0, 24)])
@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_attention_forced_plans(ht, split, mode):
    m = dsa()
    prob = workload("attention_case", fmt="bf16", B=5, H=64, n_ctx=3000, n_idx=700, pad="shuffled",
                    n_pad=40, sink=True)
    say(f"attention forced plan ht={ht} split={split} {mode}")
    try:
        m.dsa_launch_override(ht, split)
        out, lse = run_attention(prob, mode=mode)
    finally:
        m.dsa_launch_override(0, 0)
    _check_all(prob, out, lse)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("H,B", [(16, 2), (64, 2), (64, 16)])
def test_attention_late_score_jumps(mode, H, B):
    """Listed rows whose scores jump far above the running maximum late in the list: by about
    12, 45 and 150 in base-2 units (averaged over the heads) in blocks 20, 40 and 60 of the 64
    (the lazy rescale of the online softmax, taken when a maximum grows by more than 2^8, and
    the split merge across partials whose maxima differ by as much). A jumping row keeps its
    value columns and gets a multiple of the request's mean query head in its RoPE columns, so
    its score rises in every head while the outputs stay of the usual size. Random rows alone
    never grow a maximum past the first block. In decode, 16 rows x 64 heads take the 8-wave
    64-head workgroups with splits, 2 rows the 16-head ones."""
    import dataclasses
    prob = workload("attention_case", fmt="bf16", B=B, H=H, n_ctx=3000, n_idx=2048, pad="tail",
                    n_pad=0, seed=11)
    data = prob.kv.data.copy()
    r0 = prob.d_v                                                        # first RoPE column
    for b in range(prob.T):
        q = oracle.bf16_to_f64(prob.q[b])[:, r0:]                        # [H, d_rope]
        qm = q.mean(axis=0)
        per_unit = float((q @ qm).mean()) * prob.softmax_scale / np.log(2.0)
        for pos, jump in ((20 * 32 + 5, 12.0), (40 * 32 + 17, 45.0), (60 * 32 + 3, 150.0)):
            slot = int(oracle.slots_of(prob.kv, b, np.array([prob.idx_main[b, pos]]))[0])
            data[slot, r0:] = to_bf16_bits((jump / per_unit) * qm)
    prob = dataclasses.replace(prob, kv=dataclasses.replace(prob.kv, data=data))
    say("attention late score jumps", mode, H, B)
    out, lse = run_attention(prob, mode=mode)
    _check_all(prob, out, lse)
