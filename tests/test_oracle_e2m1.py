"""Pins for the oracle's FP4 E2M1 decoding and per-channel scaled gather.

torch has the packed dtype but no conversion for it, so the table is pinned
to the published value set of the OCP FP4 element (0, 0.5, 1, 1.5, 2, 3, 4, 6
and their negatives), to the positions that set fixes for each code, and to
the nibble order of a packed byte.
"""
import math

import numpy as np
import pytest

from oracle import attention, e2m1


MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.mark.parametrize("code,expected", list(enumerate(MAGNITUDES))
                         + [(8 + c, -m) for c, m in enumerate(MAGNITUDES)])
def test_e2m1_every_code(code, expected):
    v = e2m1.value(code)
    assert v == expected
    assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0)


def test_e2m1_table_properties():
    t = e2m1.table()
    assert np.all(np.diff(t[:8]) > 0)          # ascending positive half
    assert np.array_equal(t[8:], -t[:8])       # sign bit only flips the sign
    # exponent step: codes 2k+2 and 2k+4 differ by a factor 2 for normal codes
    assert t[4] == 2 * t[2] and t[6] == 2 * t[4]


def test_e2m1_packed_nibble_order():
    b = np.array([[0x21, 0xF7, 0x08]], dtype=np.uint8)
    got = e2m1.decode_packed(b)
    assert got.shape == (1, 6)
    assert np.array_equal(got[0], [0.5, 1.0, 6.0, -6.0, -0.0, 0.0])
    assert math.copysign(1.0, got[0, 4]) == -1.0


def test_e2m1_gather_applies_per_channel_scales():
    # one page of 2 tokens, 2 KV heads, head_dim 4 (2 bytes per row)
    kv = np.zeros((1, 2, 2, 2, 2), np.uint8)
    kv[0, 0, 0, 1] = [0x21, 0x43]   # K token 0 head 1: 0.5 1 1.5 2
    kv[0, 0, 1, 1] = [0x76, 0xF8]   # K token 1 head 1: 4 6 -0 -6
    kv[0, 1, 0, 1] = [0x12, 0x34]   # V token 0 head 1: 1 0.5 2 1.5
    kv[0, 1, 1, 1] = [0x99, 0x00]   # V token 1 head 1: -0.5 -0.5 0 0
    ks = np.ones((2, 4), np.float32)
    vs = np.ones((2, 4), np.float32)
    ks[1] = [2.0, 0.25, 1.0, 0.5]
    vs[1] = [1.0, 2.0, 4.0, 8.0]
    K, V = attention.gather_request(kv, [0, 1], [0], [2], 0, 1, "e2m1", ks, vs)
    assert np.array_equal(K, [[1.0, 0.25, 1.5, 1.0], [8.0, 1.5, -0.0, -3.0]])
    assert np.array_equal(V, [[1.0, 1.0, 8.0, 12.0], [-0.5, -1.0, 0.0, 0.0]])


def test_e2m1_decode_matches_hand_softmax():
    # one request, one token of K/V: the output is V itself, lse is the score
    kv = np.zeros((1, 2, 1, 1, 2), np.uint8)
    kv[0, 0, 0, 0] = [0x22, 0x22]   # K = 1 1 1 1 (times scale)
    kv[0, 1, 0, 0] = [0x7A, 0x01]   # V = -1 6 0.5 0
    ks = np.full((1, 4), 0.5, np.float32)
    vs = np.array([[3.0, 0.5, 2.0, 1.0]], np.float32)
    q = np.array([[[1.0, 2.0, 3.0, 4.0]]], np.float32)
    out, lse = attention.decode(q, kv, [0, 1], [0], [1], num_kv_heads=1, q_dtype="f32",
                                kv_dtype="e2m1", sm_scale=0.5, k_scale=ks, v_scale=vs)
    assert np.array_equal(out[0, 0], [-3.0, 3.0, 1.0, 0.0])
    assert lse[0, 0] == pytest.approx(0.5 * (0.5 * 10.0))   # sm_scale * q.k, natural log


def test_workload_encoder_rounds_to_nearest_even_and_saturates():
    """The synthetic inputs' E2M1 encoder: decode(encode(x)) is the nearest
    grid value (brute force over the 16 codes), ties go to the even code, and
    magnitudes beyond 6 saturate."""
    from workloads.synthetic import _e2m1_codes, _pack_nibbles
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * 3).astype(np.float32)
    codes = _e2m1_codes(x)
    t = e2m1.table()
    got = t[codes]
    brute = t[np.argmin(np.abs(x[:, None].astype(np.float64) - t[None, :]), axis=1)]
    assert np.array_equal(np.abs(got), np.abs(brute))
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.75, -5.0], np.float32)
    assert np.array_equal(t[_e2m1_codes(ties)], [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -1.0,
                                                 -4.0])
    packed = _pack_nibbles(_e2m1_codes(np.array([[0.5, 1.0, 6.0, -6.0]], np.float32)))
    assert np.array_equal(packed, [[0x21, 0xF7]])
