"""CPU oracle of the GQA-to-SAGA key-head merge (the closed-form initialisation).

TEST INFRASTRUCTURE. Only the tests and the benchmark's CPU-baseline leg may import
this module. The library and its binding never do, and this module shares no code
with them.

Plain float64 numpy from the exact input values. Library primitives used as single
steps: matrix products, the pseudo-inverse of a symmetric matrix and a Frobenius
norm. The pairing is found by enumerating every perfect matching.

What it follows (the paper "More Value per Key: Asymmetric Sparse Attention for
Faster LLM Decoding", as summarised on the picx.dev page DRD92V, section
"GQA-to-SAGA Conversion > Stage 1: Closed-Form Initialization"):
  * eq. (1): queries and keys are linear maps of the hidden states, Q^j = X W_Q^j
    and K^a = X W_K^a, with W_Q^j, W_K^a of shape [D, d];
  * eq. (13): the loss of replacing teacher key heads a and b by one merged key
    projection M is the squared Frobenius error of the logits Q^j (X M)^T against
    Q^j (X W_K^a)^T summed over the query heads j of head a, plus the same for b;
  * Lemma 4.1, eq. (15): the minimising M is (W_K^a S_a + W_K^b S_b)(S_a + S_b)^+
    with S_r the sum over the query heads j of head r of (Q^j)^T Q^j and + the
    Moore-Penrose pseudo-inverse;
  * Theorem 4.2 and eq. (14): the pairing of the teacher heads is a minimum-weight
    perfect matching of the complete graph whose edge (a, b) weighs eq. (13) at the
    merged projection of eq. (15).

Readings taken where the pages leave a step open (each one is a documented
parameter):
  * heads are merged in pairs (m = 2), as the indices of eq. (14) imply; the
    teacher's key-head count is even;
  * query head j belongs to teacher key head floor(j * h_k / h_q) (contiguous
    groups); after the merge the query heads of a and b both read merged head i;
  * the pseudo-inverse treats eigenvalues of S_a + S_b below rcond times the
    largest as zero, rcond = 1e-5 (the pages name no cut; it is far below the
    spectrum of a full-rank Gram of many calibration tokens and far above the
    rounding noise of a zero eigenvalue computed in fp32);
  * queries carry no position encoding (the pages' objective is on the logits of
    eq. (2) of the calibration tokens' own projections).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

RCOND = 1e-5


def query_heads_of(r: int, h_q: int, h_k: int) -> List[int]:
    """The query heads j with floor(j * h_k / h_q) == r (contiguous groups)."""
    return [j for j in range(h_q) if (j * h_k) // h_q == r]


def head_block(W: np.ndarray, i: int, d: int) -> np.ndarray:
    """Head i's projection [D, d] from a stacked projection [D, heads * d]."""
    return np.asarray(W, np.float64)[:, i * d:(i + 1) * d]


def gram_of_queries(X: np.ndarray, W_Q: np.ndarray, heads: List[int], d: int) -> np.ndarray:
    """S_r = sum over the query heads j of head r of (Q^j)^T Q^j, Q^j = X W_Q^j."""
    X = np.asarray(X, np.float64)
    S = np.zeros((d, d))
    for j in heads:
        Qj = X @ head_block(W_Q, j, d)
        S += Qj.T @ Qj
    return S


def merged_key_projection(W_a: np.ndarray, W_b: np.ndarray, S_a: np.ndarray, S_b: np.ndarray,
                          rcond: float = RCOND) -> np.ndarray:
    """Lemma 4.1, eq. (15): (W_a S_a + W_b S_b)(S_a + S_b)^+, shape [D, d]."""
    P = np.linalg.pinv(S_a + S_b, rcond=rcond, hermitian=True)
    return (W_a @ S_a + W_b @ S_b) @ P


def pair_loss(X: np.ndarray, W_Q: np.ndarray, heads_a: List[int], heads_b: List[int], W_a: np.ndarray,
              W_b: np.ndarray, M: np.ndarray, d: int) -> float:
    """Eq. (13): sum over j of head a of ||Q^j (X M)^T - Q^j (X W_a)^T||_F^2, plus the
    same over the query heads of head b with W_b."""
    X = np.asarray(X, np.float64)
    XM = X @ M
    total = 0.0
    for heads, W in ((heads_a, W_a), (heads_b, W_b)):
        XW = X @ W
        for j in heads:
            Qj = X @ head_block(W_Q, j, d)
            total += float(np.linalg.norm(Qj @ XM.T - Qj @ XW.T, "fro") ** 2)
    return total


@dataclass
class PairTable:
    """Eq. (13) at eq. (15) for every pair of teacher key heads."""
    loss: np.ndarray    # [h_k, h_k] float64, symmetric; diagonal NaN
    merged: dict        # (a, b) with a < b -> M [D, d]


def pair_table(X, W_Q, W_K, h_q: int, h_k: int, d: int, rcond: float = RCOND) -> PairTable:
    """All pairwise merge losses. W_Q [D, h_q d] and W_K [D, h_k d] stack the heads'
    projections side by side (the pages' orientation: keys are X W)."""
    S = [gram_of_queries(X, W_Q, query_heads_of(r, h_q, h_k), d) for r in range(h_k)]
    loss = np.full((h_k, h_k), np.nan)
    merged = {}
    for a in range(h_k):
        for b in range(a + 1, h_k):
            W_a, W_b = head_block(W_K, a, d), head_block(W_K, b, d)
            M = merged_key_projection(W_a, W_b, S[a], S[b], rcond)
            loss[a, b] = loss[b, a] = pair_loss(X, W_Q, query_heads_of(a, h_q, h_k),
                                                query_heads_of(b, h_q, h_k), W_a, W_b, M, d)
            merged[(a, b)] = M
    return PairTable(loss, merged)


def perfect_matchings(vertices: List[int]):
    """Every perfect matching of the complete graph on `vertices` (an even count), as
    lists of pairs (a, b) with a < b: the first vertex is paired with each other one
    in turn, then the rest is matched recursively."""
    if not vertices:
        yield []
        return
    first, rest = vertices[0], vertices[1:]
    for i, partner in enumerate(rest):
        for tail in perfect_matchings(rest[:i] + rest[i + 1:]):
            yield [(first, partner)] + tail


def min_weight_perfect_matching(w: np.ndarray) -> Tuple[List[Tuple[int, int]], float]:
    """Theorem 4.2: the perfect matching of least total weight (ties: the first one
    enumerated). Returns (pairs sorted by their first head, total weight)."""
    n = w.shape[0]
    if n % 2:
        raise ValueError("an even number of key heads is needed to merge them in pairs")
    best, best_w = None, np.inf
    for m in perfect_matchings(list(range(n))):
        tw = sum(float(w[a, b]) for a, b in m)
        if tw < best_w:
            best, best_w = m, tw
    return sorted(best), best_w


@dataclass
class Conversion:
    pairs: List[Tuple[int, int]]   # merged head i replaces teacher heads pairs[i]
    W_K: np.ndarray                # [D, (h_k / 2) d], merged projections side by side
    loss: float                    # eq. (14) at the optimum
    table: PairTable


def convert(X, W_Q, W_K, h_q: int, h_k: int, d: int, rcond: float = RCOND) -> Conversion:
    """Eq. (14): pair the teacher's key heads by Theorem 4.2 and merge each pair by
    Lemma 4.1."""
    t = pair_table(X, W_Q, W_K, h_q, h_k, d, rcond)
    pairs, total = min_weight_perfect_matching(t.loss)
    W = np.concatenate([t.merged[p] for p in pairs], axis=1)
    return Conversion(pairs, W, total, t)
