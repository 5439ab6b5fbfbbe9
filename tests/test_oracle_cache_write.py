"""Pins of the cache-write oracle (CPU): the e4m3 encoder, the UE8M0 exponent rule and the
three row packers, checked against a library cast, brute force and exact round-trip bounds."""
import numpy as np
import pytest
import torch

from oracle import cache_write as CW
from oracle.dsa_oracle import FP8_E4M3FN, ue8m0_to_f64


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_cast_on_values_midpoints_and_random():
    vals = FP8_E4M3FN[:0x7F]                      # non-negative finite values in code order
    mids = (vals[:-1] + vals[1:]) / 2             # every tie between neighbours
    rng = np.random.default_rng(0)
    rnd = rng.uniform(-448, 448, 20000) * rng.choice([1, 1e-2, 1e-4], 20000)
    x = np.concatenate([vals, -vals, mids, -mids, rnd]).astype(np.float32)
    assert np.array_equal(CW.fp8_e4m3fn_encode(x), _torch_e4m3(x))


def test_encode_saturates_and_decodes_back():
    assert list(CW.fp8_e4m3fn_encode([448, 449, 1e6, -1e6, -448.5])) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(CW.fp8_e4m3fn_encode(FP8_E4M3FN[codes]), codes)   # decode then encode


def test_ue8m0_exponent_is_the_smallest_sufficient_power():
    rng = np.random.default_rng(1)
    amax = np.concatenate([rng.lognormal(0, 8, 3000), [448.0, 448.0 * 2 ** 5, 448 * 2.0 ** -3 * 1.0000001,
                                                       1.0, 1e-38, 3.0e38]]).astype(np.float32)
    e = CW.ue8m0_exponent(amax)
    for a, ei in zip(amax.astype(np.float64), e):
        k = -200
        while 448.0 * 2.0 ** k < a:
            k += 1
        assert ei == min(max(k + 127, 1), 254), (a, ei, k)
    assert CW.ue8m0_exponent(np.float32(0.0)) == 127


def _bf16(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)   # truncation is fine here


def test_uniform_rows_round_trip_within_half_an_e4m3_step():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 576)).astype(np.float32) * rng.lognormal(0, 3, (40, 1)).astype(np.float32)
    x[3, 64:128] = 0.0                            # an all-zero group
    bits = _bf16(x)
    q, s = CW.write_uniform(bits)
    xf = CW.bf16_bits_to_f32(bits).astype(np.float64).reshape(40, 9, 64)
    back = FP8_E4M3FN[q].reshape(40, 9, 64) * s[:, :, None]
    assert s[3, 1] == 1.0 and np.all(q.reshape(40, 9, 64)[3, 1] == 0)
    # |e4m3(y) - y| <= 2^-4 |y| for normal y (3 mantissa bits), plus the subnormal step 2^-10
    err = np.abs(back - xf)
    assert np.all(err <= 2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * s[:, :, None] + 1e-30)
    amax = np.abs(xf).max(axis=2)
    nz = amax > 0
    assert np.all(np.abs(FP8_E4M3FN[q].reshape(40, 9, 64)).max(axis=2)[nz] <= 448)
    assert np.allclose(s[nz], (amax[nz] / 448).astype(np.float32), rtol=2e-7)


def test_index_key_rows_have_one_scale_per_token():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    q, s = CW.write_index_keys(_bf16(x))
    assert s.shape == (16,)
    q2, s2 = CW.quant_fp32_scaled(CW.bf16_bits_to_f32(_bf16(x)), 128)
    assert np.array_equal(q, q2) and np.array_equal(s, s2[:, 0])
    # the largest magnitude of every row lands on 448 exactly (amax / (amax / 448) rounds back)
    assert np.all(np.abs(FP8_E4M3FN[q]).max(axis=1) == 448)


def test_ds_mla_rows_layout_exponents_and_round_trip():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((24, 512)).astype(np.float32) * rng.lognormal(0, 4, (24, 1)).astype(np.float32)
    x[5, :64] = 0.0
    bits = _bf16(x)
    data, sc = CW.write_ds_mla(bits)
    assert data.shape == (24, 576) and sc.shape == (24, 8) and np.all(sc[:, 7] == 0)
    # RoPE bytes are the bf16 bits, little-endian
    assert np.array_equal(data[:, 448:].view(np.uint16), bits[:, 448:])
    assert sc[5, 0] == 127 and np.all(data[5, :64] == 0)
    xf = CW.bf16_bits_to_f32(bits).astype(np.float64)[:, :448].reshape(24, 7, 64)
    scale = ue8m0_to_f64(sc[:, :7])
    back = FP8_E4M3FN[data[:, :448]].reshape(24, 7, 64) * scale[:, :, None]
    assert np.all(np.abs(back - xf) <= 2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * scale[:, :, None])
    # the scaled group maximum lies in (224, 448]: 2^k is the smallest sufficient power
    amax = np.abs(xf).max(axis=2)
    nz = amax > 0
    r = amax[nz] / scale[nz]
    assert np.all((r > 224) & (r <= 448))


@pytest.mark.parametrize("mistake", ["ties_away", "no_saturation"])
def test_planted_encoder_mistakes_are_caught(mistake):
    vals = FP8_E4M3FN[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    if mistake == "ties_away":
        idx = np.searchsorted(vals, mids)                  # always the upper neighbour
        wrong = idx.astype(np.uint8)
        assert not np.array_equal(wrong, CW.fp8_e4m3fn_encode(mids))
    else:
        assert CW.fp8_e4m3fn_encode([500.0])[0] == 0x7E    # not 0x7F (NaN)
