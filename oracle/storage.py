"""Exact widening of stored q/K/V values to float64.

Every stored format here is a subset of float64, so widening is exact:

* ``"f32"``  — IEEE binary32 -> binary64.
* ``"f16"``  — IEEE binary16 -> binary64.
* ``"bf16"`` — the 16 stored bits are the top half of a binary32 pattern:
  ``uint16 -> uint32 << 16 -> float32 -> float64``.
* ``"e4m3"`` — the OCP E4M3FN table of ``oracle.e4m3``, then multiplied by the
  fp32 scale of its (page, KV head); the product of an 4-bit-mantissa value and
  a 24-bit-mantissa scale is exact in float64. The scale granularity — one per
  page and KV head, or one per token and KV head (the page's "per-token"
  row-wise scaling), separately for K and V — is the reading taken for the
  fp8 KV cache with scaling factors of "FlashInfer vs FlashAttention-3: GPU
  Kernel Optimization & FP8 Serving Latency", §"Production War Story".

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import numpy as np

from . import e4m3


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values (no scale) -> float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        return e4m3.decode(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")
