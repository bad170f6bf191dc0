"""CPU oracle of the SAGA + Atop-N single-token decode step.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the entry module and the
CPU-baseline leg of the benchmark may import this module. The library and its
binding never do, and this module shares no code with them.

Everything is plain float64 numpy computed from the exact input values (every
bfloat16 and float32 input value is exact in float64). Library primitives used as
single steps: a matrix-vector product, a sort, exp and a sum. No blocking,
fusion or reordering beyond the definitions.

What it follows (the paper "More Value per Key: Asymmetric Sparse Attention for
Faster LLM Decoding", as summarised on the picx.dev page DRD92V):
  * section "Attention Mechanism Formalization", eq. (2)-(4): A = q K^T / sqrt(d),
    P = softmax(A), O = P V;
  * section "Top-N Attention", eq. (6): per row of A, the indices of its N largest
    entries; every other entry is masked before the softmax;
  * section "Methodology > Atop-N Attention", steps 1-2: the N-th largest value of a
    row is used as a threshold and entries are kept by elementwise comparison; the
    exact threshold is recomputed only once every n decode steps and reused in
    between; eq. (7): O = softmax(A[i]) V[i] over the kept entries;
  * section "SAGA Architecture": key and value head counts differ (h_k != h_v);
    each query head reads the key head and the value head of its group.

Readings taken where the pages are silent (each one is a documented parameter):
  * the threshold is on the scaled logits A, compared with >=, and every entry
    tied with the threshold is kept (so a row can keep more than N entries);
  * refresh happens at steps t with t % n == 0 (t = 0 included) from that step's
    own logits, and the threshold is reused for the next n - 1 steps;
  * keys appended after the last refresh are compared with the stale threshold;
  * a stale threshold that keeps nothing forces an exact refresh of that row at
    that step (the softmax of an empty set is undefined);
  * N >= l_kv gives threshold -inf, i.e. dense attention;
  * query head j reads key head floor(j*h_k/h_q) and value head floor(j*h_v/h_q);
  * scale = 1/sqrt(d) unless given, d the query/key head dimension; thresholds are
    per (sequence, query head);
  * the value head dimension d_v may differ from d (section "Training from
    Scratch" compares a key head dimension below the value head dimension); the
    output rows then have d_v entries;
  * l_kv[b] == 0 gives O = 0, an empty selection and an unchanged threshold.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np


def key_head_of(j: int, h_q: int, h_k: int) -> int:
    """Key head read by query head j (contiguous groups of h_q/h_k query heads)."""
    return (j * h_k) // h_q


def value_head_of(j: int, h_q: int, h_v: int) -> int:
    """Value head read by query head j (contiguous groups of h_q/h_v query heads)."""
    return (j * h_v) // h_q


def attention_logits(q_j: np.ndarray, K_g: np.ndarray, scale: float) -> np.ndarray:
    """Eq. (2) for one query row: A_i = (q . K_i) * scale over the l_kv cached keys."""
    return (np.asarray(K_g, np.float64) @ np.asarray(q_j, np.float64)) * scale


def nth_largest(a: np.ndarray, N: int) -> float:
    """The exact Atop-N threshold: the N-th largest entry of row `a`, counting
    repeated values; -inf when N >= len(a) so that every entry is kept."""
    if N < 1:
        raise ValueError("N must be >= 1")
    if N >= a.size:
        return -np.inf
    return float(np.sort(a)[::-1][N - 1])


def threshold_select(a: np.ndarray, tau: float) -> np.ndarray:
    """Atop-N step 1: keep every entry whose logit is >= the threshold (sorted indices)."""
    return np.flatnonzero(a >= tau)


def sparse_softmax_pv(a_sel: np.ndarray, V_sel: np.ndarray):
    """Eq. (7): softmax over the kept logits, then the weighted sum of the kept value
    rows. Returns (o, sum of the kept probabilities)."""
    m = a_sel.max()
    w = np.exp(a_sel - m)
    p = w / w.sum()
    return p @ V_sel, float(p.sum())


@dataclass
class DecodeResult:
    O: np.ndarray                 # [B, h_q, d_v] float64
    tau: np.ndarray               # [B, h_q] float64, threshold state after the step
    sel: List[List[np.ndarray]]   # sel[b][j] = sorted kept indices
    logits: List[List[np.ndarray]]  # logits[b][j] = A[b, j, :l_kv[b]]
    sum_p: np.ndarray             # [B, h_q] sum of kept probabilities
    refreshed: np.ndarray         # [B, h_q] bool: exact threshold computed this step
    fallback: np.ndarray          # [B, h_q] bool: forced refresh (stale threshold kept nothing)


def saga_decode_step(q, K, V, l_kv, N: int, refresh_period: int, step: int,
                     tau_in: Optional[np.ndarray] = None, scale: Optional[float] = None,
                     keep_logits: bool = True) -> DecodeResult:
    """One SAGA + Atop-N decode step for a batch.

    q [B, h_q, d], K [B, h_k, L_max, d], V [B, h_v, L_max, d_v], l_kv [B].
    `tau_in` [B, h_q] is the threshold carried from the last refresh (ignored at a
    refresh step). Returns the output, the new threshold state and the selections.
    """
    q = np.asarray(q, np.float64)
    B, h_q, d = q.shape
    h_k, h_v = K.shape[1], V.shape[1]
    if h_q % h_k or h_q % h_v:
        raise ValueError("h_q must be a multiple of h_k and of h_v")
    if refresh_period < 1:
        raise ValueError("refresh period must be >= 1")
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    refresh = (step % refresh_period) == 0
    tau_prev = np.full((B, h_q), np.nan) if tau_in is None else np.asarray(tau_in, np.float64)
    if not refresh and tau_in is None:
        raise ValueError("a stale step needs the carried threshold")

    O = np.zeros((B, h_q, V.shape[3]))
    tau = tau_prev.copy()
    sum_p = np.zeros((B, h_q))
    refreshed = np.zeros((B, h_q), bool)
    fallback = np.zeros((B, h_q), bool)
    sel = [[np.zeros(0, np.int64) for _ in range(h_q)] for _ in range(B)]
    logits = [[np.zeros(0) for _ in range(h_q)] for _ in range(B)]
    for b in range(B):
        L = int(l_kv[b])
        for j in range(h_q):
            if L == 0:
                continue
            g, v = key_head_of(j, h_q, h_k), value_head_of(j, h_q, h_v)
            a = attention_logits(q[b, j], K[b, g, :L], scale)
            if refresh:
                t = nth_largest(a, N)
                refreshed[b, j] = True
            else:
                t = tau_prev[b, j]
            idx = threshold_select(a, t)
            if idx.size == 0:
                t = nth_largest(a, N)
                idx = threshold_select(a, t)
                refreshed[b, j] = fallback[b, j] = True
            O[b, j], sum_p[b, j] = sparse_softmax_pv(a[idx], np.asarray(V[b, v, idx], np.float64))
            tau[b, j] = t
            sel[b][j] = idx
            if keep_logits:
                logits[b][j] = a
    return DecodeResult(O, tau, sel, logits, sum_p, refreshed, fallback)


def refresh_threshold(q, K, l_kv, N: int, scale: Optional[float] = None):
    """The exact threshold alone: tau[b, j] = N-th largest of A[b, j, :l_kv[b]]
    (NaN for an empty row, which has no threshold)."""
    q = np.asarray(q, np.float64)
    B, h_q, d = q.shape
    h_k = K.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    tau = np.full((B, h_q), np.nan)
    for b in range(B):
        L = int(l_kv[b])
        for j in range(h_q):
            if L:
                tau[b, j] = nth_largest(attention_logits(q[b, j], K[b, key_head_of(j, h_q, h_k), :L], scale), N)
    return tau


def dense_gqa(q, K, V, l_kv, scale: Optional[float] = None) -> np.ndarray:
    """Eq. (2)-(4) for one decode token: softmax over every cached key, then the full
    P V product, with query head j reading key head g(j) and value head v(j). With
    h_k == h_v this is grouped-query attention (the pages' dense baseline); with
    h_k < h_v it is SAGA with full attention (section "SAGA Architecture" without
    the Atop-N selection)."""
    q = np.asarray(q, np.float64)
    B, h_q, d = q.shape
    h_k, h_v = K.shape[1], V.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    O = np.zeros((B, h_q, V.shape[3]))
    for b in range(B):
        L = int(l_kv[b])
        if L == 0:
            continue
        for j in range(h_q):
            a = attention_logits(q[b, j], K[b, key_head_of(j, h_q, h_k), :L], scale)
            O[b, j], _ = sparse_softmax_pv(a, np.asarray(V[b, value_head_of(j, h_q, h_v), :L], np.float64))
    return O
