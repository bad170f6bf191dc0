"""Byte accounting of one decode-attention step (used for the roofline figures).

The vector-read count follows the worked example of the learnaivisually.com
explainer "SAGA attention" (its one-layer, one-decode-step read table): dense
attention reads h_kv * l_kv key vectors and as many value vectors; with top-N the
value side drops to h_q * N vectors while the key side still reads h_k * l_kv.

The algorithmic bytes of this library's sparse step count what the method cannot
avoid: every cached key of the h_k key heads, plus the selected value rows. A
selected row shared by several query heads of one value head is counted once
(the union), which is the conservative figure; the explainer's per-query-head
count is reported beside it.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence


def vector_reads(h_q: int, h_k: int, h_v: int, l_kv: int, N: Optional[int] = None):
    """(key vectors, value vectors, total) read by one layer for one decode token.

    N=None is dense attention (every value row of every value head); otherwise each
    query head reads N value rows.
    """
    keys = h_k * l_kv
    values = h_v * l_kv if N is None else h_q * min(N, l_kv)
    return keys, values, keys + values


def key_bytes(h_k: int, d: int, l_kv: Iterable[int], elem_bytes: int) -> int:
    """Bytes of the key cache one step streams: sum_b l_kv[b] * h_k * d * s."""
    return sum(int(L) for L in l_kv) * h_k * d * elem_bytes


def dense_bytes(h_kv: int, d: int, l_kv: Iterable[int], elem_bytes: int) -> int:
    """Bytes one dense GQA step streams: every key and value row of h_kv heads."""
    return 2 * sum(int(L) for L in l_kv) * h_kv * d * elem_bytes


def selected_value_bytes(union_rows: Sequence[int], d: int, elem_bytes: int) -> int:
    """Bytes of the value rows gathered, given the number of distinct selected rows
    per (sequence, value head)."""
    return sum(int(r) for r in union_rows) * d * elem_bytes
