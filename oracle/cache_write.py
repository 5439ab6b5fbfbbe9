"""CPU oracle of the cache-write step: bf16 rows -> the fp8 cache formats the layer reads.

TEST INFRASTRUCTURE ONLY (imported by tests/; never by the HIP library or its binding; it
shares no code with them).

The formats are those of aiter PR 4382 "Paged Sparse Attention Gluon Kernel" (section
"Supported formats & dtypes"): the uniform 2D fp8 pool (fp8 e4m3 values with one fp32 scale
per 64 channels) and the packed fp8_ds_mla token (448 NoPE channels as fp8 with one UE8M0
power-of-two exponent per 64 channels, then the 64 RoPE channels as bf16, 584 bytes per token,
the data and exponents of a page stored apart); and the fp8 index keys with one fp32 scale per
token. The pages give the layouts and the OCP e4m3 flavour, not the rounding of the scales;
the readings taken here:

* values are rounded to e4m3 to nearest, ties to even, after saturating to +-448; the fnuz
  flavour of the uniform pool (section "fp8 flavors": bias 8) saturates to +-240, and zero of
  either sign is byte 0x00 (0x80 is NaN there);
* fp32 scales: scale = amax / 448 (fnuz: amax / 240) in fp32 arithmetic (1.0 for an all-zero
  group), and each value is divided by its scale in fp32 before rounding;
* UE8M0 exponents: the smallest integer k with 448 * 2^k >= amax (exact), stored as k + 127
  clamped to [1, 254]; an all-zero group stores 127 (scale 1). Dividing by 2^k is exact.

All arithmetic that decides a byte is done on float32 values exactly as stated (numpy float32
division is IEEE round-to-nearest), the rounding to e4m3 exactly (float64 on values that are
exact in float32).
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def _e4m3fn_finite_values() -> tuple[np.ndarray, np.ndarray]:
    """Non-negative finite e4m3fn values in increasing order with their codes (OCP: bias 7,
    exponent field 0 is subnormal m/8 * 2^-6, S.1111.111 is NaN, no infinities)."""
    vals, codes = [], []
    for code in range(0x7F):             # 0x7F is NaN
        e, m = code >> 3, code & 7
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(v)
        codes.append(code)
    return np.asarray(vals, np.float64), np.asarray(codes, np.uint8)


_POS_VALS, _POS_CODES = _e4m3fn_finite_values()


def fp8_e4m3fn_encode(x) -> np.ndarray:
    """float values -> OCP e4m3fn bytes: saturate to +-448, round to nearest, ties to the even
    code (even mantissa LSB). Zero (of either sign) encodes as +0 or -0 by sign."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), FP8_MAX)
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[hi] & 1) == 0) & (hi != lo))
    exact = _POS_VALS[hi] == a
    idx = np.where(exact | pick_hi, hi, lo)
    code = _POS_CODES[idx].astype(np.uint8)
    return np.where(sign, code | 0x80, code).astype(np.uint8)


def _e4m3fnuz_finite_values() -> tuple[np.ndarray, np.ndarray]:
    """Non-negative fnuz e4m3 values in increasing order with their codes (bias 8, exponent
    field 0 is subnormal m/8 * 2^-7, every code 0x00..0x7F finite: the largest is 240)."""
    vals = [(m / 8.0) * 2.0 ** -7 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 8)
            for e, m in ((c >> 3, c & 7) for c in range(0x80))]
    return np.asarray(vals, np.float64), np.arange(0x80, dtype=np.uint8)


_FNUZ_VALS, _FNUZ_CODES = _e4m3fnuz_finite_values()
FP8_FNUZ_MAX = 240.0


def fp8_e4m3fnuz_encode(x) -> np.ndarray:
    """float values -> fnuz e4m3 bytes: saturate to +-240, round to nearest, ties to the even
    code; a value that rounds to zero is 0x00 whatever its sign (there is no negative zero)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP8_FNUZ_MAX)
    hi = np.minimum(np.searchsorted(_FNUZ_VALS, a, side="left"), len(_FNUZ_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _FNUZ_VALS[lo]
    dhi = _FNUZ_VALS[hi] - a
    pick_hi = (_FNUZ_VALS[hi] == a) | (dhi < dlo) | ((dhi == dlo) & ((_FNUZ_CODES[hi] & 1) == 0) & (hi != lo))
    code = _FNUZ_CODES[np.where(pick_hi, hi, lo)].astype(np.uint8)
    neg = np.signbit(x) & (code != 0)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def bf16_bits_to_f32(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def ue8m0_exponent(amax) -> np.ndarray:
    """Stored exponent byte for group maxima amax (float32, >= 0): k + 127 for the smallest
    integer k with 448 * 2^k >= amax, clamped to [1, 254]; 127 for amax = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, 127, dtype=np.int64)
    nz = amax > 0
    m, e = np.frexp(amax[nz])            # amax = m * 2^e, m in [0.5, 1)
    # 448 * 2^k >= amax  <=>  2^k >= amax / 448; with amax = (2m) * 2^(e-1), 448 = 1.75 * 2^8:
    # k = e - 9 if 2m <= 1.75 else e - 8
    k = np.where(2.0 * m <= 1.75, e - 9, e - 8)
    out[nz] = k + 127
    return np.clip(out, 1, 254)


def quant_fp32_scaled(values_f32: np.ndarray, group: int, fnuz: bool = False):
    """float32 [n, D] -> (e4m3 bytes [n, D], float32 scales [n, D // group]) with one scale per
    group of `group` channels: scale = amax / 448 (fp32), byte = e4m3(x / scale) (fp32 divide);
    fnuz: amax / 240 and the fnuz encoding."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    n, D = v.shape
    g = v.reshape(n, D // group, group)
    amax = np.abs(g).max(axis=2)
    fmax = np.float32(FP8_FNUZ_MAX if fnuz else FP8_MAX)
    scale = np.where(amax > 0, amax / fmax, np.float32(1.0)).astype(np.float32)
    q = (g / scale[:, :, None]).astype(np.float32)          # IEEE float32 division
    enc = fp8_e4m3fnuz_encode if fnuz else fp8_e4m3fn_encode
    return enc(q).reshape(n, D), scale


def write_uniform(src_bf16_bits: np.ndarray, fnuz: bool = False):
    """bf16 rows [n, D] -> uniform pool rows: (fp8 bytes [n, D], fp32 scales [n, D / 64]),
    OCP or fnuz bytes."""
    return quant_fp32_scaled(bf16_bits_to_f32(src_bf16_bits), 64, fnuz)


def write_index_keys(src_bf16_bits: np.ndarray):
    """bf16 index keys [n, di] -> (fp8 bytes [n, di], fp32 per-token scale [n])."""
    q, s = quant_fp32_scaled(bf16_bits_to_f32(src_bf16_bits), src_bf16_bits.shape[1])
    return q, s[:, 0]


def write_ds_mla(src_bf16_bits: np.ndarray, d_nope: int = 448, d_rope: int = 64):
    """bf16 rows [n, 512] (448 NoPE + 64 RoPE) -> (token data [n, 576] bytes: NoPE fp8 then the
    RoPE bf16 bytes little-endian, exponent bytes [n, 8]: 7 UE8M0 bytes then 0)."""
    bits = np.ascontiguousarray(src_bf16_bits, dtype=np.uint16)
    n = bits.shape[0]
    v = bf16_bits_to_f32(bits)
    nope = v[:, :d_nope].reshape(n, d_nope // 64, 64)
    amax = np.abs(nope).max(axis=2)
    e = ue8m0_exponent(amax)
    scale = np.ldexp(1.0, e - 127)                            # exact powers of two
    q = fp8_e4m3fn_encode(nope.astype(np.float64) / scale[:, :, None]).reshape(n, d_nope)
    rope = bits[:, d_nope:d_nope + d_rope].view(np.uint8).reshape(n, 2 * d_rope)
    data = np.concatenate([q, rope], axis=1)
    sc = np.zeros((n, 8), dtype=np.uint8)
    sc[:, : d_nope // 64] = e.astype(np.uint8)
    return data, sc
