"""OCP FP8 E4M3FN decoding, written from the bit formula.

The pages name the fp8 KV format only as E4M3 ("FlashInfer vs
FlashAttention-3: GPU Kernel Optimization & FP8 Serving Latency", §"Production
War Story: The FP8 Precision Underflow Failure", and the ``fp8_mode`` field of
its §"Multi-File Production Implementation" config). The reading taken is the
OCP E4M3FN encoding: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals when the exponent field is 0, no infinities, and NaN only for
``S.1111.111`` (0x7F / 0xFF). The largest finite magnitude is 448.

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import math

import numpy as np

BIAS = 7


def value(byte: int) -> float:
    """Real value of one E4M3FN byte (float, exact)."""
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    exp_field = (byte >> 3) & 0xF
    mant = byte & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        # subnormal: 0.mmm * 2^(1 - bias)
        return sign * (mant / 8.0) * 2.0 ** (1 - BIAS)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - BIAS)


def table() -> np.ndarray:
    """float64 ``[256]`` lookup: byte -> value."""
    return np.array([value(b) for b in range(256)], dtype=np.float64)


_TABLE = table()


def decode(bytes_: np.ndarray) -> np.ndarray:
    """Elementwise E4M3FN bytes (uint8 array) -> float64 values."""
    return _TABLE[np.asarray(bytes_, dtype=np.uint8)]
