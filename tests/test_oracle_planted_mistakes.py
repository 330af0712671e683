"""The oracle's pins must catch plausible mistakes.

Each test plants one mistake in a copy of an oracle function (on the CPU, via
monkeypatch) and checks that an independent pin then fails.
"""
import math

import numpy as np
import pytest

from oracle import attention, e4m3, merge, storage
from workloads import custom_workload, host_case

from test_oracle_attention import brute_force


def _case():
    w = custom_workload(3, 4, 2, 8, 4, "f32", "f32", [9, 16, 3], pool_pages=12)
    return host_case(w, 7, poison=True), w


def _matches_brute(case, w):
    out, lse = attention.decode_case(case)
    bo, bl = brute_force(case, w.scale())
    return (np.all(np.isfinite(out)) and np.allclose(out, bo, rtol=1e-12, atol=1e-12)
            and np.allclose(lse, bl, rtol=1e-12, atol=1e-12))


def test_unmodified_oracle_passes():
    case, w = _case()
    assert _matches_brute(case, w)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    case, w = _case()
    real = attention.gather_request

    def wrong(kv, indptr, indices, last, r, kv_head, *a, **k):
        return real(kv, indptr, indices, last, r, (kv_head + 1) % kv.shape[3], *a, **k)

    monkeypatch.setattr(attention, "gather_request", wrong)
    assert not _matches_brute(case, w)


def test_wrong_slot_index_is_caught(monkeypatch):
    case, w = _case()

    def wrong(indptr, indices, last, P, r):
        L = attention.request_length(indptr, last, P, r)
        t = np.arange(L)
        pages = np.asarray(indices[indptr[r]:indptr[r + 1]], dtype=np.int64)
        return pages[t // P], (t + 1) % P

    monkeypatch.setattr(attention, "token_locations", wrong)
    assert not _matches_brute(case, w)


def test_untruncated_last_page_is_caught(monkeypatch):
    case, w = _case()
    monkeypatch.setattr(attention, "request_length",
                        lambda indptr, last, P, r: (int(indptr[r + 1]) - int(indptr[r])) * P)
    with np.errstate(invalid="ignore"):
        assert not _matches_brute(case, w)


def test_missing_scale_is_caught(monkeypatch):
    case, w = _case()
    real = attention.attend
    monkeypatch.setattr(attention, "attend", lambda qh, K, V, s: real(qh, K, V, 1.0))
    assert not _matches_brute(case, w)


def test_transposed_kv_halves_are_caught(monkeypatch):
    case, w = _case()
    real = attention.gather_request

    def swapped(*a, **k):
        K, V = real(*a, **k)
        return V, K

    monkeypatch.setattr(attention, "gather_request", swapped)
    assert not _matches_brute(case, w)


def test_normalised_o_in_merge_is_caught(monkeypatch):
    """Weighting o by d as well (as if o were normalised) breaks split == unsplit."""
    def wrong(a, b):
        m_a, d_a, o_a = a
        m_b, d_b, o_b = b
        if m_a == -math.inf:
            return b
        if m_b == -math.inf:
            return a
        m = max(m_a, m_b)
        wa, wb = d_a * math.exp(m_a - m), d_b * math.exp(m_b - m)
        return (m, wa + wb, o_a * wa + o_b * wb)

    monkeypatch.setattr(merge, "merge", wrong)
    rng = np.random.default_rng(0)
    s, V = rng.standard_normal(20), rng.standard_normal((20, 4))
    o, _ = merge.finalize(merge.fold([merge.chunk_state(s[:9], V[:9]),
                                      merge.chunk_state(s[9:], V[9:])], 4))
    wts = np.exp(s - s.max())
    assert not np.allclose(o, (wts @ V) / wts.sum(), rtol=1e-9)


def test_wrong_e4m3_bias_is_caught(monkeypatch):
    monkeypatch.setattr(e4m3, "BIAS", 8)
    assert e4m3.value(0x38) != 1.0 and e4m3.value(0x7E) != 448.0


def test_wrong_bf16_shift_is_caught(monkeypatch):
    """A widening that shifts the stored bits by 15 instead of 16 fails the
    bf16 pins (torch's own bfloat16 conversion and the known patterns)."""
    import test_oracle_e4m3_storage as pins
    real = storage.widen

    def wrong(x, dtype):
        if dtype == "bf16":
            bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
            return bits.view(np.float32).astype(np.float64)
        return real(x, dtype)

    monkeypatch.setattr(storage, "widen", wrong)
    for pin in (pins.test_bf16_widening_matches_torch, pins.test_bf16_widening_known_patterns):
        with pytest.raises(AssertionError):
            pin()


# Plausible mistakes in the partition rule, each a one-place edit of the
# oracle's own source: (text in oracle/plan.py, its replacement).
PLAN_MUTANTS = {
    "tie_break_to_largest_k": ("cost < best_cost", "cost <= best_cost"),
    "cost_without_start_term": ("+ 2 * min_chunk_pages)", "+ 0 * min_chunk_pages)"),
    "waves_over_slots_not_compute_units": ("_ceil_div(slots, max(1, slots_per_cu))", "slots"),
    "near_equal_test_without_slack": ("8 * N * units <= 9 * S", "N * units <= S"),
    "share_without_kv_heads": ("_ceil_div(S * num_kv_heads, slots * balance)",
                               "_ceil_div(S, slots * balance)"),
    "no_last_page_trim": ("kv_len -= page_size - last[r]", "kv_len -= 0"),
    "shortest_first": ("rows.sort(key=lambda t: (-t[3],", "rows.sort(key=lambda t: (t[3],"),
    "partial_slot_off_by_one": ("slot = merge_indptr[r] + c * nq[r]",
                                "slot = merge_indptr[r] + 1 + c * nq[r]"),
}


def _mutant_plan(name):
    import os
    import types

    from oracle import plan as oplan
    old, new = PLAN_MUTANTS[name]
    with open(os.path.join(os.path.dirname(oplan.__file__), "plan.py")) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutant {name}: the text to edit must occur once"
    mod = types.ModuleType(f"plan_mutant_{name}")
    exec(compile(src.replace(old, new), f"<oracle.plan mutant {name}>", "exec"), mod.__dict__)
    return mod.plan


@pytest.mark.parametrize("mutant", sorted(PLAN_MUTANTS))
def test_plan_mutants_are_caught(mutant, monkeypatch):
    """oracle.plan replaced by a mutated copy: the hand-worked partitions or the
    seeded invariants (chunk length by enumeration, coverage, token counts,
    partial slots, order) must then fail."""
    from oracle import plan as oplan

    import test_oracle_plan as pins
    monkeypatch.setattr(oplan, "plan", _mutant_plan(mutant))
    failed = 0
    hand = [pins.test_hand_worked_partitions, pins.test_hand_worked_multi_query_partitions,
            pins.test_cost_ties_take_the_fewest_chunks, pins.test_uniform_batch_is_cut_to_fill_the_device,
            pins.test_waves_count_compute_units_not_slots,
            pins.test_uniform_batch_just_over_the_device_is_cut_into_waves]
    for pin in hand + [lambda s=s: pins.check_partition(s) for s in pins.SEEDS]:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught the {mutant} mutant"


def test_rowwise_scale_slot_mixup_is_caught():
    """Indexing a row-wise scale by the wrong slot must break the brute-force match."""
    w = custom_workload(3, 4, 2, 8, 4, "e4m3", "bf16", [9, 16, 3], pool_pages=12,
                        kv_scale="token")
    case = host_case(w, 7, poison=True)
    assert _matches_brute(case, w)
    wrong = dict(case)
    wrong["k_scale"] = np.roll(case["k_scale"], 1, axis=2)  # scale of the neighbouring slot
    out, _ = attention.decode_case(wrong)
    bo, _ = brute_force(case, w.scale())
    assert not np.allclose(out, bo, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("mistake", ["unsigned", "offset_binary", "high_nibble_first"])
def test_int4_decoding_mistakes_are_caught(mistake, monkeypatch):
    """A plausible misreading of the int4 codes (no sign extension, an
    offset-binary code, the high nibble first) fails the int4 pins."""
    from oracle import int4
    if mistake == "unsigned":
        monkeypatch.setattr(int4, "_TABLE", np.arange(16, dtype=np.float64))
    elif mistake == "offset_binary":
        monkeypatch.setattr(int4, "_TABLE", np.arange(16, dtype=np.float64) - 8)
    else:
        t = int4.table()
        monkeypatch.setattr(int4, "decode_packed", lambda b: np.stack(
            [t[np.asarray(b) >> 4], t[np.asarray(b) & 0xF]], axis=-1).reshape(
                np.asarray(b).shape[:-1] + (-1,)))
    got = int4.decode_packed(np.array([[0x8F, 0x70, 0x19]], np.uint8))[0]
    assert not np.array_equal(got, [-1.0, -8.0, 0.0, 7.0, -7.0, 1.0])
