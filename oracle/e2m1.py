"""OCP FP4 E2M1 decoding, written from the bit formula.

"FlashInfer vs FlashAttention-3: GPU Kernel Optimization & FP8 Serving
Latency" names FP4 PageAttention with per-channel scaling factors
(§"Decision Matrix: Choosing the Right Attention Engine", the custom KV-cache
quantization case) but no encoding.
The reading taken is the OCP MX FP4 element E2M1: 1 sign bit, 2 exponent bits
with bias 1, 1 mantissa bit, a subnormal when the exponent field is 0, no
infinities and no NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. Two elements
share a byte, the lower-indexed one in the low nibble.

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import numpy as np

BIAS = 1


def value(nibble: int) -> float:
    """Real value of one E2M1 code (float, exact)."""
    nibble = int(nibble) & 0xF
    sign = -1.0 if nibble & 0x8 else 1.0
    exp_field = (nibble >> 1) & 0x3
    mant = nibble & 0x1
    if exp_field == 0:
        return sign * (mant / 2.0) * 2.0 ** (1 - BIAS)  # subnormal: 0.m * 2^(1 - bias)
    return sign * (1.0 + mant / 2.0) * 2.0 ** (exp_field - BIAS)


def table() -> np.ndarray:
    """float64 ``[16]`` lookup: code -> value."""
    return np.array([value(c) for c in range(16)], dtype=np.float64)


_TABLE = table()


def decode_packed(bytes_: np.ndarray) -> np.ndarray:
    """Packed bytes ``[..., n]`` -> float64 values ``[..., 2n]`` (element 2i
    from the low nibble of byte i, element 2i+1 from the high nibble)."""
    b = np.asarray(bytes_, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.float64)
    out[..., 0::2] = _TABLE[b & 0xF]
    out[..., 1::2] = _TABLE[b >> 4]
    return out
