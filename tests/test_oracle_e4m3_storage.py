"""Pins for the oracle's storage decoding (E4M3FN table, bf16 widening)."""
import math

import numpy as np
import pytest
import torch

from oracle import e4m3, storage


@pytest.mark.parametrize("byte,expected", [
    (0x00, 0.0),
    (0x80, -0.0),
    (0x01, 2.0 ** -9),        # smallest subnormal
    (0x07, 7 * 2.0 ** -9),    # largest subnormal
    (0x08, 2.0 ** -6),        # smallest normal
    (0x38, 1.0),              # exponent field 7 == bias
    (0x3C, 1.5),
    (0x7E, 448.0),            # largest finite
    (0xFE, -448.0),
    (0x40, 2.0),
])
def test_e4m3_special_values(byte, expected):
    v = e4m3.value(byte)
    assert v == expected
    assert math.copysign(1.0, v) == math.copysign(1.0, expected)


@pytest.mark.parametrize("byte", [0x7F, 0xFF])
def test_e4m3_nan(byte):
    assert math.isnan(e4m3.value(byte))


def test_e4m3_table_matches_torch_float8_e4m3fn():
    raw = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = raw.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def test_e4m3_positive_half_strictly_increasing():
    t = e4m3.table()[:0x7F]
    assert np.all(np.diff(t) > 0)


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint64).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = storage.widen(bits, "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def test_bf16_widening_known_patterns():
    assert storage.widen(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    assert storage.widen(np.array([0xC000], np.uint16), "bf16")[0] == -2.0
    assert storage.widen(np.array([0x0001], np.uint16), "bf16")[0] == 2.0 ** -133


def test_f32_widening_exact():
    x = np.array([1.0, 2.0 ** -149, 3.4028234663852886e38, -0.1], np.float32)
    assert np.array_equal(storage.widen(x, "f32"), x.astype(np.float64))
