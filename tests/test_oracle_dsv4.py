"""Pins of the oracle's DeepSeek-V4 options (CPU only): the fnuz e4m3 flavour of the uniform
pool (decode table, encoder, pool rows) and the attention sink / base-2 lse.

The fnuz table and encoder are tied to torch's float8_e4m3fnuz cast (a library routine) and to
the OCP table through the bias difference; the sink is tied to the plain softmax definition by
an identity (a sink is a listed row whose value columns are zero and whose logit is the sink);
the base-2 lse to closed forms. test_planted_sink_mistakes_are_caught plants slips in the
oracle and checks that these pins notice.
"""
import math

import numpy as np
import pytest
import torch

from oracle import cache_write as CW
from oracle import dsa_oracle as O
from workloads import gen as G


def _bf16(x):
    return G.to_bf16_bits(np.asarray(x, np.float32))


def _problem(q, rows, d_v, scale, sink=None, lse_log2=False):
    q = np.asarray(q, np.float32)
    rows = np.asarray(rows, np.float32)
    D = rows.shape[1]
    kv = G.KVPool("bf16", _bf16(rows), None, 1, None, np.zeros(1, np.int32), D, 0)
    return G.DSAProblem(name="pin", T=1, H=q.shape[0], d_qk=D, d_v=d_v, topk=rows.shape[0],
                        q=_bf16(q)[None], kv=kv, row_req=np.zeros(1, np.int32),
                        row_len=np.array([rows.shape[0]], np.int32), n_req=1, softmax_scale=scale,
                        sink=sink, lse_log2=lse_log2)


# --------------------------------------------------------------------------- fnuz bytes

def test_fnuz_table_matches_torch_cast_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fnuz).to(torch.float64).numpy()
    t = O.FP8_E4M3FNUZ
    nan = np.isnan(ref)
    assert np.flatnonzero(nan).tolist() == [0x80] and np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])


def test_fnuz_is_half_of_ocp_apart_from_the_ends():
    """Bias 8 against bias 7 on the same bits: every shared finite code halves; 0x7F / 0xFF are
    +-240 (NaN in OCP) and 0x80 is NaN (-0 in OCP)."""
    codes = [c for c in range(256) if c not in (0x7F, 0xFF, 0x80)]
    assert np.array_equal(O.FP8_E4M3FNUZ[codes], O.FP8_E4M3FN[codes] / 2)
    assert O.FP8_E4M3FNUZ[0x7F] == 240.0 and O.FP8_E4M3FNUZ[0xFF] == -240.0
    assert O.FP8_E4M3FNUZ[0x01] == 2.0 ** -10                # smallest subnormal


def test_fnuz_encoder_matches_torch_cast():
    vals = O.FP8_E4M3FNUZ[:0x80]
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(0)
    rnd = rng.uniform(-240, 240, 20000) * rng.choice([1, 1e-2, 1e-4], 20000)
    edge = [300.0, -300.0, 240.5, 232.0, -232.0, 232.01, -0.0, -1e-9, 2.0 ** -11, -(2.0 ** -11),
            3 * 2.0 ** -12, 1e-30]
    x = np.concatenate([vals, -vals, mids, -mids, rnd, edge]).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -240, 240)).to(torch.float8_e4m3fnuz).view(torch.uint8).numpy()
    got = CW.fp8_e4m3fnuz_encode(x)
    assert np.array_equal(got, ref)
    assert not np.any(got == 0x80)                            # never the NaN byte


def test_fnuz_generator_rows_decode_within_rounding():
    """Uniform fnuz rows decode to the values the generator quantised within half a step:
    2^-4 relative for normals, 2^-11 of the group scale for subnormals (step 2^-10)."""
    vals = G._normal(5, 98, (256, 512))
    data, sc = G.quant_uniform(vals, fnuz=True)
    pool = G.KVPool("fp8_uniform_fnuz", data, sc, 1, None, np.zeros(1, np.int32), 448, 64)
    dec = O.kv_rows(pool, 0, np.arange(256))
    scale = np.repeat(sc.astype(np.float64), 64, 1)
    ref = vals.astype(np.float64)
    assert np.all(np.abs(dec - ref) <= 2.0 ** -4 * np.abs(ref) + scale * 2.0 ** -11)
    assert np.allclose(np.abs(dec / scale).reshape(256, 8, 64).max(2), 240.0)


def test_fnuz_writer_round_trip_and_group_maximum():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((32, 512)).astype(np.float32) * rng.lognormal(0, 3, (32, 1)).astype(np.float32)
    x[2, :64] = 0.0
    x[3, 64:128] = -0.0
    bits = _bf16(x)
    q, s = CW.write_uniform(bits, fnuz=True)
    assert not np.any(q == 0x80)
    xf = CW.bf16_bits_to_f32(bits).astype(np.float64).reshape(32, 8, 64)
    back = O.FP8_E4M3FNUZ[q].reshape(32, 8, 64) * s[:, :, None]
    assert np.all(np.abs(back - xf) <= 2.0 ** -4 * np.abs(xf) + 2.0 ** -11 * s[:, :, None])
    nz = np.abs(xf).max(2) > 0
    assert np.all(np.abs(O.FP8_E4M3FNUZ[q].reshape(32, 8, 64)).max(2)[nz] == 240.0)
    assert s[2, 0] == 1.0 and s[3, 1] == 1.0 and np.all(q.reshape(32, 8, 64)[[2, 3], [0, 1]] == 0)


def test_fnuz_nan_byte_in_a_cache_is_an_error():
    data = np.zeros((2, 128), np.uint8)
    data[1, 5] = 0x80
    pool = G.KVPool("fp8_uniform_fnuz", data, np.ones((2, 2), np.float32), 1, None,
                    np.zeros(1, np.int32), 64, 64)
    O.kv_rows(pool, 0, np.array([0]))
    with pytest.raises(ValueError):
        O.kv_rows(pool, 0, np.array([1]))


# --------------------------------------------------------------------------- sink and base-2 lse

def _sink_case(seed=1, H=4, n=20):
    """A 576-wide problem (value = first 512 columns) and a virtual row r* whose value columns
    are zero: its logit for head h is scale * q[h, 512:] . r*[512:], used as head h's sink."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, 576)).astype(np.float32)
    rows = rng.standard_normal((n, 576)).astype(np.float32)
    star = np.zeros(576, np.float32)
    star[512:] = 2.0 * rng.standard_normal(64)
    scale = 1 / math.sqrt(576)
    qb = O.bf16_to_f64(_bf16(q))
    sink = scale * (qb[:, 512:] @ O.bf16_to_f64(_bf16(star))[512:])
    return q, rows, star, scale, sink


def test_sink_equals_a_listed_zero_value_row():
    q, rows, star, scale, sink = _sink_case()
    lst = np.array([3, -1, 7, 0, 19, 11])
    out, lse = O.attention_row(_problem(q, rows, 512, scale, sink=sink), 0, lst)
    plain = _problem(q, np.vstack([rows, star]), 512, scale)
    out_ref, lse_ref = O.attention_row(plain, 0, np.append(lst, len(rows)))
    assert np.allclose(out, out_ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)
    # and it changes the result: the sink takes a visible share of the mass
    out0, lse0 = O.attention_row(_problem(q, rows, 512, scale), 0, lst)
    assert np.abs(out - out0).max() > 1e-3 and np.all(lse > lse0)


def test_sink_special_values():
    q, rows, star, scale, sink = _sink_case(seed=2)
    lst = np.array([1, 2, 3])
    # empty list: out 0, lse = the sink (natural log or base 2)
    oute, lsee = O.attention_row(_problem(q, rows, 512, scale, sink=sink), 0, np.full(5, -1))
    assert np.all(oute == 0) and np.array_equal(lsee, sink)
    _, lsee2 = O.attention_row(_problem(q, rows, 512, scale, sink=sink, lse_log2=True), 0, np.full(5, -1))
    assert np.allclose(lsee2, sink / math.log(2), rtol=1e-15)
    # a -inf sink is no sink
    none = O.attention_row(_problem(q, rows, 512, scale), 0, lst)
    ninf = O.attention_row(_problem(q, rows, 512, scale, sink=np.full(4, -np.inf)), 0, lst)
    assert np.array_equal(none[0], ninf[0]) and np.array_equal(none[1], ninf[1])
    # a sink far above every logit takes all the mass
    big = np.full(4, 1.0e4)
    outb, lseb = O.attention_row(_problem(q, rows, 512, scale, sink=big), 0, lst)
    assert np.all(np.abs(outb) < 1e-300) and np.allclose(lseb, big, rtol=1e-15)


def test_lse_base2_closed_forms():
    """A zero query gives every logit 0: with one row listed n times (each listed entry
    counts) lse = ln n, base 2: log2 n; a sink of ln 8 beside 8 such entries doubles the mass."""
    rows = np.random.default_rng(3).standard_normal((5, 64)).astype(np.float32)
    q = np.zeros((2, 64), np.float32)
    lst = np.full(8, 4)
    _, l_e = O.attention_row(_problem(q, rows, 64, 0.7), 0, lst)
    _, l_2 = O.attention_row(_problem(q, rows, 64, 0.7, lse_log2=True), 0, lst)
    assert np.allclose(l_e, math.log(8), rtol=1e-15) and np.allclose(l_2, 3.0, rtol=1e-15)
    out_s, l_s = O.attention_row(_problem(q, rows, 64, 0.7, sink=np.full(2, math.log(8)), lse_log2=True), 0, lst)
    assert np.allclose(l_s, 4.0, rtol=1e-15)
    assert np.allclose(out_s, 0.5 * O.bf16_to_f64(_bf16(rows))[4], rtol=1e-14)


def _sink_pins_pass():
    try:
        test_sink_equals_a_listed_zero_value_row()
        test_sink_special_values()
        test_lse_base2_closed_forms()
    except AssertionError:
        return False
    return True


def test_planted_sink_mistakes_are_caught(monkeypatch):
    assert _sink_pins_pass()
    real = O.attention_row

    def sink_only_in_lse(prob, t, a, b=None):
        out, lse = real(prob, t, a, b)
        s = prob.sink
        prob.sink = None
        try:
            out, _ = real(prob, t, a, b)
        finally:
            prob.sink = s
        return out, lse

    def natural_log_always(prob, t, a, b=None):
        flag = prob.lse_log2
        prob.lse_log2 = False
        try:
            return real(prob, t, a, b)
        finally:
            prob.lse_log2 = flag

    def sink_times_scale(prob, t, a, b=None):
        s = prob.sink
        prob.sink = None if s is None else np.asarray(s) * prob.softmax_scale
        try:
            return real(prob, t, a, b)
        finally:
            prob.sink = s

    for fake in (sink_only_in_lse, natural_log_always, sink_times_scale):
        with monkeypatch.context() as m:
            m.setattr(O, "attention_row", fake)
            assert not _sink_pins_pass(), f"planted mistake {fake.__name__} went unnoticed"
