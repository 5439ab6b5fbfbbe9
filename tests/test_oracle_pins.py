"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties one part of the oracle to a hand-derived worked value, a closed form, an
invariant, or an independent library routine, chosen so that a plausible slip (a dropped
ReLU, a wrong sign, a transposed operand, an off-by-one page index, a wrong exponent bias)
fails at least one of them. test_planted_mistakes_are_caught plants such slips in the oracle
and checks that the pins notice.
"""
import heapq
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import dsa_oracle as O
from workloads import gen as G

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(x):
    return G.to_bf16_bits(np.asarray(x, dtype=np.float32))


def _score_problem(q_idx, w, keys, page_size=1, block_table=None, key_dtype="bf16", scale=None,
                   index_scale=1.0):
    q_idx = np.asarray(q_idx, np.float32)[None]
    keys = np.asarray(keys, np.float32)
    n = keys.shape[0] if block_table is None else keys.shape[0]
    if key_dtype == "bf16":
        kp = G.KeyPool("bf16", _bf16(keys), None, page_size,
                       None if block_table is None else np.asarray(block_table, np.int32),
                       np.zeros(1, np.int32) if block_table is None else None)
    else:
        kp = G.KeyPool("fp8", keys.astype(np.uint8), np.asarray(scale, np.float32), page_size,
                       None if block_table is None else np.asarray(block_table, np.int32),
                       np.zeros(1, np.int32) if block_table is None else None)
    kv = G.KVPool("bf16", np.zeros((max(n, 1), 2), np.uint16), None, 1, None, np.zeros(1, np.int32), 1, 1)
    return G.DSAProblem(name="pin", T=1, H=1, d_qk=2, d_v=2, topk=1, q=np.zeros((1, 1, 2), np.uint16),
                        kv=kv, row_req=np.zeros(1, np.int32), row_len=np.array([n], np.int32), n_req=1,
                        softmax_scale=1.0, Hi=q_idx.shape[1], di=q_idx.shape[2], q_idx=_bf16(q_idx),
                        w=np.asarray(w, np.float32)[None], kpool=kp, index_scale=index_scale)


def _attn_problem(q, rows, d_v=None, scale=1.0, fmt="bf16"):
    q = np.asarray(q, np.float32)
    if q.ndim == 1:
        q = q[None]
    rows = np.asarray(rows, np.float32)
    D = rows.shape[1]
    kv = G.KVPool("bf16", _bf16(rows), None, 1, None, np.zeros(1, np.int32), D, 0)
    return G.DSAProblem(name="pin", T=1, H=q.shape[0], d_qk=D, d_v=d_v or D, topk=rows.shape[0],
                        q=_bf16(q)[None], kv=kv, row_req=np.zeros(1, np.int32),
                        row_len=np.array([rows.shape[0]], np.int32), n_req=1, softmax_scale=scale)


# --------------------------------------------------------------------------- stored formats

def test_fp8_table_matches_torch_cast_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = O.FP8_E4M3FN
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]


def test_fp8_table_golden_spot_values():
    g = _load("fp8_e4m3fn_spot.json")
    for v in g["values"]:
        assert O.FP8_E4M3FN[int(v["byte"], 16)] == v["value"], v
    for b in g["nan_bytes"]:
        assert math.isnan(O.FP8_E4M3FN[int(b, 16)])
    assert math.copysign(1.0, O.FP8_E4M3FN[0x80]) == -1.0


def test_ue8m0_closed_form():
    assert O.ue8m0_to_f64(np.array([127]))[0] == 1.0
    assert O.ue8m0_to_f64(np.array([128]))[0] == 2.0
    assert O.ue8m0_to_f64(np.array([120]))[0] == 1.0 / 128
    assert O.ue8m0_to_f64(np.array([0]))[0] == 2.0 ** -127
    assert O.ue8m0_to_f64(np.array([254]))[0] == 2.0 ** 127
    with pytest.raises(ValueError):
        O.ue8m0_to_f64(np.array([255]))


def test_bf16_widening_known_patterns_and_torch():
    pats = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000], np.uint16)
    v = O.bf16_to_f64(pats)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 3.140625
    assert v[3] == 2.0 ** -133 and v[4] == (2 - 2 ** -7) * 2.0 ** 127
    rnd = np.random.default_rng(5).integers(0, 1 << 16, 4096).astype(np.uint16)
    rnd = rnd[(rnd & 0x7F80) != 0x7F80]   # skip inf/nan patterns
    ref = torch.from_numpy(rnd.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_to_f64(rnd), ref)


# --------------------------------------------------------------------------- addressing

def test_slots_closed_form_page_table():
    pool = G.KeyPool("bf16", np.zeros((12, 1), np.uint16), None, 4, np.array([[2, 0, 1]], np.int32), None)
    got = O.slots_of(pool, 0, np.arange(12))
    assert got.tolist() == [8, 9, 10, 11, 0, 1, 2, 3, 4, 5, 6, 7]
    packed = G.KeyPool("bf16", np.zeros((12, 1), np.uint16), None, 1, None, np.array([0, 7], np.int32))
    assert O.slots_of(packed, 1, np.arange(3)).tolist() == [7, 8, 9]


def test_ds_mla_addressing_hand_built_page():
    """Bytes placed at the page's documented offsets, read back through the oracle."""
    blk = 4
    n_pages = 2
    page_bytes = blk * 584
    data = np.zeros((n_pages, page_bytes), np.uint8)
    # token (page 1, pos 2): NoPE byte c = fp8 0x38 (1.0) for c in group g, exponent 127 + g
    page, pos = 1, 2
    for c in range(448):
        data[page, pos * 576 + c] = 0x38 if c % 2 == 0 else 0xB8   # +1 / -1
    for g in range(7):
        data[page, blk * 576 + pos * 8 + g] = 127 + g
    data[page, blk * 576 + pos * 8 + 7] = 255          # the pad byte is never read as a scale
    for i in range(64):                                 # RoPE i = bf16(i - 10), little endian
        b = int(_bf16([i - 10.0])[0])
        data[page, pos * 576 + 448 + 2 * i] = b & 0xFF
        data[page, pos * 576 + 448 + 2 * i + 1] = b >> 8
    # all other tokens: exponent 127 so they decode cleanly
    for p in range(n_pages):
        for t in range(blk):
            if (p, t) != (page, pos):
                data[p, blk * 576 + t * 8: blk * 576 + t * 8 + 7] = 127
    pool = G.KVPool("fp8_ds_mla", data, None, blk, np.array([[0, 1]], np.int32), None, 448, 64)
    row = O.kv_rows(pool, 0, np.array([blk + pos]))[0]      # logical blk+pos -> page 1, pos 2
    exp_nope = np.array([(1.0 if c % 2 == 0 else -1.0) * 2.0 ** (c // 64) for c in range(448)])
    assert np.array_equal(row[:448], exp_nope)
    assert np.array_equal(row[448:], np.arange(64) - 10.0)


def test_uniform_pool_hand_built():
    D = 128
    data = np.full((3, D), 0x38, np.uint8)       # 1.0 everywhere
    data[1, 70] = 0x40                           # 2.0
    scales = np.array([[1, 1], [0.5, 3.0], [1, 1]], np.float32)
    pool = G.KVPool("fp8_uniform", data, scales, 1, None, np.zeros(1, np.int32), 64, 64)
    row = O.kv_rows(pool, 0, np.array([1]))[0]
    exp = np.concatenate([np.full(64, 0.5), np.full(64, 3.0)])
    exp[70] = 6.0
    assert np.array_equal(row, exp)


@pytest.mark.parametrize("fmt", ["fp8_ds_mla", "fp8_uniform"])
def test_generator_quantisation_round_trip(fmt):
    """Decoded rows match the float values the generator quantised, within e4m3's rounding
    bound (half an ulp: 2^-4 relative for normals, 2^-10 of the group scale for subnormals)."""
    vals = G._normal(3, 99, (512, 512))
    if fmt == "fp8_ds_mla":
        pool = G.KVPool(fmt, G.pack_ds_mla(vals, 256), None, 256, None, np.zeros(1, np.int32), 448, 64)
        dec = O.kv_rows(pool, 0, np.arange(512))
        nope, ref = dec[:, :448], vals[:, :448].astype(np.float64)
        scale = np.repeat(2.0 ** np.ceil(np.log2(np.abs(vals[:, :448]).reshape(512, 7, 64).max(2) / 448.0)), 64, 1)
        assert np.all(np.abs(nope - ref) <= 2.0 ** -4 * np.abs(ref) + scale * 2.0 ** -10)
        assert np.array_equal(dec[:, 448:], O.bf16_to_f64(G.to_bf16_bits(vals[:, 448:])))
    else:
        data, sc = G.quant_uniform(vals)
        pool = G.KVPool(fmt, data, sc, 1, None, np.zeros(1, np.int32), 448, 64)
        dec = O.kv_rows(pool, 0, np.arange(512))
        scale = np.repeat(sc.astype(np.float64), 64, 1)
        ref = vals.astype(np.float64)
        assert np.all(np.abs(dec - ref) <= 2.0 ** -4 * np.abs(ref) + scale * 2.0 ** -9)


# --------------------------------------------------------------------------- scores

def test_scores_golden_worked_example():
    g = _load("index_scores_tiny.json")
    p = _score_problem(g["q_idx"], g["w"], g["keys_logical"])
    assert O.index_scores_row(p, 0).tolist() == g["expected_scores"]
    pg = g["paged"]
    pp = _score_problem(g["q_idx"], g["w"], pg["physical_keys"], page_size=pg["page_size"],
                        block_table=pg["block_table"])
    assert O.index_scores_row(pp, 0).tolist() == g["expected_scores"]


def test_scores_one_head_is_relu_of_dot():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 32)).astype(np.float32)
    keys = rng.standard_normal((50, 32)).astype(np.float32)
    p = _score_problem(q, [1.0], keys)
    qq = O.bf16_to_f64(_bf16(q))[0]
    kk = O.bf16_to_f64(_bf16(keys))
    ref = np.array([max(0.0, float(np.dot(qq, kk[s]))) for s in range(50)])
    assert np.allclose(O.index_scores_row(p, 0), ref, rtol=1e-14, atol=0)


def test_scores_all_negative_dots_are_zero_and_w_signs():
    rng = np.random.default_rng(2)
    q = np.abs(rng.standard_normal((3, 16))).astype(np.float32) + 0.1
    keys = -np.abs(rng.standard_normal((20, 16))).astype(np.float32) - 0.1
    p = _score_problem(q, [0.3, -2.0, 1.0], keys)
    assert np.all(O.index_scores_row(p, 0) == 0)
    # positive dots with a negative weight give a negative score
    p2 = _score_problem(q, [0.0, -1.0, 0.0], -keys)
    assert np.all(O.index_scores_row(p2, 0) < 0)


def test_scores_linear_in_w_and_head_permutation():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((6, 24)).astype(np.float32)
    keys = rng.standard_normal((40, 24)).astype(np.float32)
    w1 = rng.uniform(-1, 1, 6).astype(np.float32)
    w2 = rng.uniform(-1, 1, 6).astype(np.float32)
    s1 = O.index_scores_row(_score_problem(q, w1, keys), 0)
    s2 = O.index_scores_row(_score_problem(q, w2, keys), 0)
    s12 = O.index_scores_row(_score_problem(q, w1.astype(np.float64) + w2, keys), 0)
    assert np.allclose(s12, s1 + s2, rtol=1e-6, atol=1e-6)   # w1+w2 rounded to fp32
    perm = rng.permutation(6)
    sp = O.index_scores_row(_score_problem(q[perm], w1[perm], keys), 0)
    assert np.allclose(sp, s1, rtol=1e-13, atol=1e-13)
    s3 = O.index_scores_row(_score_problem(q, w1, keys, index_scale=0.125), 0)
    assert np.array_equal(s3, 0.125 * s1)


def test_scores_nonnegative_weights_give_nonnegative_scores():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((8, 16)).astype(np.float32)
    keys = rng.standard_normal((64, 16)).astype(np.float32)
    s = O.index_scores_row(_score_problem(q, rng.uniform(0, 1, 8), keys), 0)
    assert np.all(s >= 0) and np.any(s > 0)


def test_scores_fp8_keys_equal_bf16_keys_of_the_decoded_values():
    """fp8 byte * scale with a power-of-two scale is exact in bf16, so both paths must agree."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    codes = rng.integers(0, 256, (30, 32)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    scale = np.ldexp(1.0, rng.integers(-3, 4, 30)).astype(np.float32)
    p8 = _score_problem(q, [1, 0.5, 0.25, 2], codes, key_dtype="fp8", scale=scale)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy() * scale[:, None]
    pb = _score_problem(q, [1, 0.5, 0.25, 2], dec)
    assert np.array_equal(O.index_scores_row(p8, 0), O.index_scores_row(pb, 0))


# --------------------------------------------------------------------------- top-k

def test_topk_golden_worked_example():
    g = _load("index_scores_tiny.json")
    s = np.array(g["expected_scores"])
    for k, exp in g["topk"].items():
        idx, n = O.topk_row(s, int(k))
        assert idx.tolist() == exp["indices"] and n == exp["lens"]


@pytest.mark.parametrize("seed", range(5))
def test_topk_matches_heapq_nlargest(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    s = np.round(rng.standard_normal(n) * 4) / 4      # plenty of exact ties
    k = int(rng.integers(1, 500))
    idx, m = O.topk_row(s, k)
    ref = heapq.nlargest(min(k, n), range(n), key=lambda i: (s[i], -i))
    assert idx[:m].tolist() == ref
    assert m == min(k, n) and np.all(idx[m:] == -1)


def test_topk_defining_property_and_special_cases():
    rng = np.random.default_rng(9)
    s = rng.integers(0, 20, 300).astype(np.float64)
    idx, m = O.topk_row(s, 37)
    sel = set(idx[:m].tolist())
    rest = [i for i in range(300) if i not in sel]
    assert min(s[list(sel)]) >= max(s[rest])
    thr = min(s[list(sel)])
    # among positions scoring exactly thr, the selected ones are the smallest positions
    tied = sorted(i for i in range(300) if s[i] == thr)
    chosen = sorted(i for i in sel if s[i] == thr)
    assert chosen == tied[:len(chosen)]
    assert O.topk_row(s, 1)[0][0] == int(np.argmax(s))
    all_idx, m_all = O.topk_row(s[:10], 16)
    assert sorted(all_idx[:10].tolist()) == list(range(10)) and m_all == 10


# --------------------------------------------------------------------------- attention

def test_attention_golden_worked_example():
    g = _load("attention_tiny.json")
    p = _attn_problem(g["q"], g["rows_logical"])
    out, lse = O.attention_row(p, 0, np.array(g["list"]))
    e = math.e
    assert np.allclose(out[0], [e / (1 + e), (5 + 7 * e) / (1 + e)], rtol=1e-15)
    assert abs(lse[0] - math.log(1 + e)) < 1e-15


def test_attention_full_selection_equals_dense_sdpa():
    """topk >= context: sparse attention is dense softmax attention (torch SDPA, float64)."""
    rng = np.random.default_rng(7)
    H, n, D, d_v = 4, 33, 40, 32
    q = rng.standard_normal((H, D)).astype(np.float32)
    rows = rng.standard_normal((n, D)).astype(np.float32)
    scale = 1 / math.sqrt(D)
    p = _attn_problem(q, rows, d_v=d_v, scale=scale)
    out, lse = O.attention_row(p, 0, rng.permutation(n))
    qq = torch.from_numpy(O.bf16_to_f64(_bf16(q)))[None, :, None, :]
    kk = torch.from_numpy(O.bf16_to_f64(_bf16(rows)))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qq, kk[None, None].expand(1, H, n, D), kk[None, None, :, :d_v].expand(1, H, n, d_v), scale=scale)
    assert np.allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    from scipy.special import logsumexp
    lref = logsumexp(scale * (qq[0, :, 0].numpy() @ kk.numpy().T), axis=1)
    assert np.allclose(lse, lref, rtol=1e-13, atol=1e-13)


def test_attention_single_row_and_zero_query():
    rng = np.random.default_rng(8)
    rows = rng.standard_normal((9, 24)).astype(np.float32)
    q = rng.standard_normal((2, 24)).astype(np.float32)
    p = _attn_problem(q, rows, d_v=16, scale=0.5)
    out, lse = O.attention_row(p, 0, np.array([-1, 4, -1]))
    r4 = O.bf16_to_f64(_bf16(rows))[4]
    assert np.array_equal(out, np.stack([r4[:16], r4[:16]]))
    assert np.allclose(lse, 0.5 * O.bf16_to_f64(_bf16(q)) @ r4, rtol=1e-14)
    pz = _attn_problem(np.zeros((1, 24)), rows, d_v=24, scale=0.5)
    outz, lsez = O.attention_row(pz, 0, np.array([1, 3, 5]))
    rr = O.bf16_to_f64(_bf16(rows))
    assert np.allclose(outz[0], rr[[1, 3, 5]].mean(0), rtol=1e-14, atol=1e-15)
    assert abs(lsez[0] - math.log(3)) < 1e-15


def test_attention_padding_and_permutation_invariance():
    rng = np.random.default_rng(10)
    rows = rng.standard_normal((50, 32)).astype(np.float32)
    p = _attn_problem(rng.standard_normal((3, 32)), rows, d_v=32, scale=0.2)
    lst = rng.choice(50, 20, replace=False)
    out, lse = O.attention_row(p, 0, lst)
    padded = np.insert(lst, [0, 5, 5, 20], -1)
    out2, lse2 = O.attention_row(p, 0, rng.permutation(padded))
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-14) and np.allclose(lse, lse2, rtol=1e-14)
    oute, lsee = O.attention_row(p, 0, np.full(7, -1))
    assert np.all(oute == 0) and np.all(lsee == -np.inf)


def test_attention_two_lists_are_one_softmax_over_the_union():
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((40, 32)).astype(np.float32)
    p = _attn_problem(rng.standard_normal((2, 32)), rows, d_v=32, scale=0.3)
    p.extra_kv = p.kv   # same rows behind a second cache
    a, b = rng.choice(40, 7, replace=False), rng.choice(40, 9, replace=False)
    out, lse = O.attention_row(p, 0, a, b)
    out1, lse1 = O.attention_row(p, 0, np.concatenate([a, b]))
    assert np.allclose(out, out1, rtol=1e-13, atol=1e-14) and np.allclose(lse, lse1, rtol=1e-14)


def test_layer_one_token_segment_attends_to_itself():
    p = G.causal_prefill((9, 1), H=2, Hi=2, di=32, topk=4, d_nope=64, d_rope=32)
    r = O.layer_row(p, 9)
    row = O.bf16_to_f64(p.kv.data[9])
    assert r["lens"] == 1 and r["idx"].tolist() == [0, -1, -1, -1]
    assert np.array_equal(r["out"], np.stack([row[:64]] * 2))


def test_layer_causal_rows_see_only_their_prefix():
    p = G.causal_prefill((12, 5), H=2, Hi=4, di=32, topk=3, d_nope=64, d_rope=32)
    for t in range(p.T):
        r = O.layer_row(p, t)
        n = int(p.row_len[t])
        assert r["scores"].shape == (n,)
        assert r["lens"] == min(3, n) and np.all(r["idx"][:r["lens"]] < n)


# --------------------------------------------------------------------------- planted mistakes

def _pins_pass():
    try:
        test_scores_golden_worked_example()
        test_scores_one_head_is_relu_of_dot()
        test_scores_all_negative_dots_are_zero_and_w_signs()
        test_topk_golden_worked_example()
        test_attention_golden_worked_example()
        test_attention_full_selection_equals_dense_sdpa()
        test_attention_padding_and_permutation_invariance()
        test_ds_mla_addressing_hand_built_page()
        test_slots_closed_form_page_table()
    except AssertionError:
        return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pins_pass()

    def no_relu(prob, t):
        b, n = int(prob.row_req[t]), int(prob.row_len[t])
        keys = O.key_rows(prob.kpool, b, np.arange(n))
        return prob.w[t].astype(np.float64) @ (O.bf16_to_f64(prob.q_idx[t]) @ keys.T)

    def off_by_one_page(pool, b, positions):
        s = np.asarray(positions, dtype=np.int64)
        if pool.block_table is not None:
            P = int(pool.page_size)
            return np.asarray(pool.block_table[b], np.int64)[s // P] * P + (s + 1) % P
        return int(pool.req_base[b]) + s

    def ties_by_larger_position(scores):
        return np.lexsort((-np.arange(scores.shape[0]), -scores))

    real_attention = O.attention_row

    def no_max_shift_log2(prob, t, a, b=None):
        out, lse = real_attention(prob, t, a, b)
        return out, lse / math.log(2)   # base-2 lse

    for name, fake in [("index_scores_row", no_relu), ("slots_of", off_by_one_page),
                       ("order_key", ties_by_larger_position),
                       ("attention_row", no_max_shift_log2)]:
        with monkeypatch.context() as m:
            m.setattr(O, name, fake)
            assert not _pins_pass(), f"planted mistake in {name} went unnoticed"
