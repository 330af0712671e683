"""Pins for the oracle's int4 decoding and per-channel scaled gather.

The codes are pinned to two's complement as the integer hardware computes it
(numpy's arithmetic right shift of an int8 sign-extends the nibble), to the
values the definition fixes at its ends (0, 7, -8, -1), to the nibble order
of a packed byte, and to hand-worked gathers and decodes.
"""
import numpy as np
import pytest

from oracle import attention, int4


@pytest.mark.parametrize("nibble", range(16))
def test_int4_every_code_is_twos_complement(nibble):
    # sign extension by the integer unit: place the nibble in the top of an
    # int8 and shift it back down arithmetically
    ext = int((np.array([nibble << 4], np.uint8).view(np.int8) >> 4)[0])
    assert int4.value(nibble) == ext
    assert -8 <= int4.value(nibble) <= 7


def test_int4_table_ends_and_order():
    t = int4.table()
    assert (t[0], t[7], t[8], t[15]) == (0.0, 7.0, -8.0, -1.0)
    assert np.array_equal(t[:8], np.arange(8))           # non-negative half in order
    assert np.array_equal(t[8:], np.arange(-8, 0))       # negative half in order
    assert sorted(t.tolist()) == list(range(-8, 8))      # every integer once


def test_int4_packed_nibble_order():
    b = np.array([[0x8F, 0x70, 0x19]], dtype=np.uint8)
    got = int4.decode_packed(b)
    assert got.shape == (1, 6)
    assert np.array_equal(got[0], [-1.0, -8.0, 0.0, 7.0, -7.0, 1.0])


def test_int4_gather_applies_per_channel_scales():
    # one page of 2 tokens, 2 KV heads, head_dim 4 (2 bytes per row)
    kv = np.zeros((1, 2, 2, 2, 2), np.uint8)
    kv[0, 0, 0, 1] = [0x21, 0x43]   # K token 0 head 1: 1 2 3 4
    kv[0, 0, 1, 1] = [0x8F, 0x07]   # K token 1 head 1: -1 -8 7 0
    kv[0, 1, 0, 1] = [0x12, 0xE3]   # V token 0 head 1: 2 1 3 -2
    kv[0, 1, 1, 1] = [0x99, 0x00]   # V token 1 head 1: -7 -7 0 0
    ks = np.ones((2, 4), np.float32)
    vs = np.ones((2, 4), np.float32)
    ks[1] = [2.0, 0.25, 1.0, 0.5]
    vs[1] = [1.0, 2.0, 4.0, 8.0]
    K, V = attention.gather_request(kv, [0, 1], [0], [2], 0, 1, "i4", ks, vs)
    assert np.array_equal(K, [[2.0, 0.5, 3.0, 2.0], [-2.0, -2.0, 7.0, 0.0]])
    assert np.array_equal(V, [[2.0, 2.0, 12.0, -16.0], [-7.0, -14.0, 0.0, 0.0]])


def test_int4_decode_matches_hand_softmax():
    # two tokens, one KV head, head_dim 4; weights by hand
    kv = np.zeros((1, 2, 2, 1, 2), np.uint8)
    kv[0, 0, 0, 0] = [0x11, 0x11]   # K0 = 1 1 1 1
    kv[0, 0, 1, 0] = [0xFF, 0xFF]   # K1 = -1 -1 -1 -1
    kv[0, 1, 0, 0] = [0x0F, 0x07]   # V0 = -1 0 7 0
    kv[0, 1, 1, 0] = [0x08, 0x00]   # V1 = -8 0 0 0
    ks = np.full((1, 4), 0.5, np.float32)
    vs = np.array([[1.0, 1.0, 2.0, 1.0]], np.float32)
    q = np.array([[[1.0, 0.0, 0.0, 1.0]]], np.float32)
    out, lse = attention.decode(q, kv, [0, 1], [0], [2], num_kv_heads=1, q_dtype="f32",
                                kv_dtype="i4", sm_scale=1.0, k_scale=ks, v_scale=vs)
    # scores: q.K0 = 0.5 * 2 = 1, q.K1 = -1
    w0, w1 = np.exp(1.0), np.exp(-1.0)
    expect = (w0 * np.array([-1.0, 0.0, 14.0, 0.0]) + w1 * np.array([-8.0, 0.0, 0.0, 0.0])) / (
        w0 + w1)
    assert np.allclose(out[0, 0], expect, rtol=1e-14, atol=0)
    assert lse[0, 0] == pytest.approx(np.log(w0 + w1), rel=1e-14)


def test_workload_encoder_rounds_half_to_even_and_clips():
    """The synthetic inputs' int4 encoder: codes are the integer nearest to
    x * 7/3 (brute force over -8 .. 7, ties to the even integer), clipped,
    and packed two's complement, low nibble first."""
    from workloads.synthetic import I4_STEPS_PER_SIGMA, _pack_nibbles
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 1.5).astype(np.float32)
    y = x * np.float32(I4_STEPS_PER_SIGMA)
    codes = np.clip(np.rint(y), -8, 7).astype(np.int8)
    grid = np.arange(-8, 8, dtype=np.float64)
    d = np.abs(y[:, None].astype(np.float64) - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, grid[None, :], np.nan)
    # nearest; on a tie the even integer
    even = np.where(np.isfinite(cand) & (cand % 2 == 0), cand, np.nan)
    brute = np.where(np.isnan(even).all(axis=1), np.nanmin(cand, axis=1), np.nanmin(even, axis=1))
    assert np.array_equal(codes.astype(np.float64), brute)
    packed = _pack_nibbles(np.array([[-1, -8, 7, 0]], np.int8).view(np.uint8) & np.uint8(0xF))
    assert np.array_equal(packed, [[0x8F, 0x07]])
    assert np.array_equal(int4.decode_packed(packed)[0], [-1.0, -8.0, 7.0, 0.0])
