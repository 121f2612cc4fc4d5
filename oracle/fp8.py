"""OCP FP8 E4M3 ("E4M3FN") decoding — oracle, test infrastructure only.

The PocketLLM page ("Qwen3.8-27B-FP8", section "Implemented execution path",
and section "KV cache dtype and the 262,144-token boundary") stores the FP8
cache as E4M3 bytes with one fp16 scale per token, per KV head and per
64-channel block. The pages do not spell out the bit format; the reading here
is the OCP 8-bit floating point E4M3 encoding: 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, and S.1111.111 as the only NaN
pattern. Largest finite magnitude 448, smallest subnormal 2^-9.

Quantisation (appending new K/V rows to an FP8 cache). Reading taken (the
pages fix the layout but print no quantiser): per 64-channel block,
scale = fp16 of amax / 448 (amax = largest |x| of the block; the division in
fp32, then rounded to nearest even fp16), 1.0 for a block whose scale would
be 0; each code is the E4M3 value nearest x / scale (the division in fp32,
clamped to +-448), ties to the even code, the sign kept (-0 gives 0x80).
"""
import math

import numpy as np


def e4m3_value(code: int) -> float:
    """Value of one E4M3 byte, from the sign/exponent/mantissa fields."""
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m / 8.0, 1 - 7)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of an array of E4M3 bytes."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def dequantize(codes, scales) -> np.ndarray:
    """Dequantised float64 K or V rows: decode(code) * scale of the code's
    64-channel block. codes [..., D] uint8, scales [..., D//64] fp16."""
    vals = e4m3_decode(codes)
    sc = np.asarray(scales).astype(np.float64)
    d = vals.shape[-1]
    return vals * np.repeat(sc, 64, axis=-1)[..., :d]


# the non-negative finite E4M3 values, ascending, with their codes (0x00..0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = E4M3_TABLE[:0x7F]


def e4m3_encode(y) -> np.ndarray:
    """E4M3 bytes of values y (|y| <= 448): the nearest finite value, ties to
    the even code (mantissa bit 0 clear), found by searching the table of
    values; the sign bit is the sign of y, zeros included."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if (a > 448).any():
        raise ValueError("e4m3_encode takes |y| <= 448")
    hi = np.searchsorted(_POS_VALS, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    sign = np.signbit(y).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize_rows(x):
    """E4M3 codes and fp16 scales of rows x [..., D] (D a multiple of 64),
    per 64-channel block: (codes [..., D] uint8, scales [..., D//64] fp16)."""
    x32 = np.asarray(x, dtype=np.float32)
    d = x32.shape[-1]
    xb = x32.reshape(*x32.shape[:-1], d // 64, 64)
    amax = np.abs(xb).max(axis=-1)
    sc = (amax / np.float32(448.0)).astype(np.float32).astype(np.float16)
    sc = np.where(sc == 0, np.float16(1.0), sc)
    y = xb / sc.astype(np.float32)[..., None]          # fp32 division
    y = np.clip(y, np.float32(-448.0), np.float32(448.0))
    codes = e4m3_encode(y.astype(np.float64)).reshape(x32.shape)
    return codes, sc
