"""Partial softmax states (m, d, o) and the online-softmax merge rule.

"FlashDecoding + FlashInfer — the decode-time attention story", §"FlashDecoding
— the split-KV trick": each block of the split-KV launch produces a partial
``(m, d, o)`` for its KV chunk, and two partials combine as

    m = max(m_a, m_b)
    d = d_a * exp(m_a - m) + d_b * exp(m_b - m)
    o = o_a * exp(m_a - m) + o_b * exp(m_b - m)

with the same recurrence used per tile inside the main kernel and per split in
the reduction kernel.

Readings taken where the pages leave a step open:

* ``o`` is the unnormalised sum ``sum_t exp(s_t - m) v_t``: the rule rescales
  ``o`` by ``exp(m_a - m)`` alone, with no ``d`` weight, which is only right
  for unnormalised sums. The final output is ``o / d``.
* One token is the state ``(s_t, 1, v_t)``.
* The empty state ``(-inf, 0, 0)`` is the identity; merging it must return
  the other operand unchanged (the rule as printed would form
  ``-inf - (-inf)`` when both are empty).

Test infrastructure: see the package docstring.
"""
from __future__ import annotations

import math
from functools import reduce
from typing import Iterable, Tuple

import numpy as np

State = Tuple[float, float, np.ndarray]


def identity(head_dim: int) -> State:
    return (-math.inf, 0.0, np.zeros(head_dim))


def token_state(s_t: float, v_t: np.ndarray) -> State:
    return (float(s_t), 1.0, np.asarray(v_t, dtype=np.float64).copy())


def chunk_state(s: np.ndarray, V: np.ndarray) -> State:
    """Partial state of a chunk of scores ``s`` [n] and values ``V`` [n, D]."""
    if len(s) == 0:
        return identity(V.shape[1])
    m = float(np.max(s))
    p = np.exp(s - m)
    return (m, float(p.sum()), p @ V)


def merge(a: State, b: State) -> State:
    m_a, d_a, o_a = a
    m_b, d_b, o_b = b
    if m_a == -math.inf:
        return (m_b, d_b, np.array(o_b, dtype=np.float64))
    if m_b == -math.inf:
        return (m_a, d_a, np.array(o_a, dtype=np.float64))
    m = max(m_a, m_b)
    wa = math.exp(m_a - m)
    wb = math.exp(m_b - m)
    return (m, d_a * wa + d_b * wb, o_a * wa + o_b * wb)


def fold(states: Iterable[State], head_dim: int) -> State:
    return reduce(merge, states, identity(head_dim))


def finalize(state: State):
    """Normalised output ``o / d`` and natural-log LSE ``m + ln d``."""
    m, d, o = state
    return o / d, m + math.log(d)


def merge_normalized(v_a, lse_a, v_b, lse_b):
    """Merge two normalised attention results over disjoint token sets.

    A result ``(v, lse)`` (output row and natural-log log-sum-exp) is the state
    ``(lse, 1, v)``: ``o / d = v`` and ``m + ln d = lse``. Arrays ``v_*``
    ``[..., D]`` and ``lse_*`` ``[...]``; each row is merged with ``merge`` and
    finalised. This is how the levels of cascade attention combine.
    """
    v_a = np.asarray(v_a, dtype=np.float64)
    v_b = np.asarray(v_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    out = np.empty(np.broadcast_shapes(v_a.shape, v_b.shape))
    lse = np.empty(out.shape[:-1])
    for idx in np.ndindex(*lse.shape):
        st = merge((float(lse_a[idx]), 1.0, v_a[idx]), (float(lse_b[idx]), 1.0, v_b[idx]))
        out[idx], lse[idx] = finalize(st)
    return out, lse


def split_attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float,
                 bounds: Iterable[Tuple[int, int]]):
    """Attention of one query computed chunk by chunk and merged.

    ``bounds`` lists ``[begin, end)`` token ranges that tile ``[0, L)``.
    """
    states = []
    for b, e in bounds:
        s = sm_scale * (K[b:e] @ qh)
        states.append(chunk_state(s, V[b:e]))
    return finalize(fold(states, K.shape[1]))
