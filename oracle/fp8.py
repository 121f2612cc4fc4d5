"""OCP FP8 E4M3 ("E4M3FN") decoding — oracle, test infrastructure only.

The PocketLLM page ("Qwen3.8-27B-FP8", section "Implemented execution path",
and section "KV cache dtype and the 262,144-token boundary") stores the FP8
cache as E4M3 bytes with one fp16 scale per token, per KV head and per
64-channel block. The pages do not spell out the bit format; the reading here
is the OCP 8-bit floating point E4M3 encoding: 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, and S.1111.111 as the only NaN
pattern. Largest finite magnitude 448, smallest subnormal 2^-9.
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
