"""OCP FP8 E4M3 ("e4m3fn") decoding as a 256-entry fp64 table.

Test infrastructure only (see the package docstring).

The pages say only "FP8" (Atlas engine article, "技术深度解析" › quantisation;
GB10 article: "paged FP8 KV cache").  Reading taken: the OCP 8-bit floating
point E4M3 format -- sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
no infinities, NaN only at S.1111.111, subnormals at exponent field 0.
Every code's value is given by the closed form below, written out per code.
"""

import numpy as np


def _value_of_code(x: int) -> float:
    sign = -1.0 if (x >> 7) & 1 else 1.0
    exp_field = (x >> 3) & 0xF
    mant = x & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        # subnormal: (-1)^s * (M / 8) * 2^(1 - 7)
        return sign * mant * 2.0 ** -9
    # normal: (-1)^s * (1 + M / 8) * 2^(E - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


_TABLE = np.array([_value_of_code(x) for x in range(256)], dtype=np.float64)
_TABLE.setflags(write=False)


def decode_table() -> np.ndarray:
    """fp64 value of every byte 0..255 (read-only view)."""
    return _TABLE


def decode(codes) -> np.ndarray:
    """Decode an array of E4M3 bytes to fp64 by table lookup."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]
