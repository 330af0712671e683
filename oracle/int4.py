"""Signed 4-bit integer (int4) KV codes.

"FlashInfer vs FlashAttention-3: GPU Kernel Optimization & FP8 Serving
Latency" names int4 PageAttention with per-channel scaling factors
(§"Decision Matrix: Choosing the Right Attention Engine", the custom KV-cache
quantization case) but gives no encoding. The reading taken is the plain
signed integer of four bits in two's complement: a nibble b stands for
b - 16 when its top bit is set, else b, so codes run -8 .. 7; the stored value
is code x scale, with one scale per (KV head, channel) as for FP4. Two codes
share a byte, the lower-indexed one in the low nibble.

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import numpy as np


def value(nibble: int) -> int:
    """Integer of one two's-complement nibble."""
    nibble = int(nibble) & 0xF
    return nibble - 16 if nibble & 0x8 else nibble


def table() -> np.ndarray:
    """float64 ``[16]`` lookup: nibble -> integer value."""
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
