"""Pins of the key-head merge oracle (GQA-to-SAGA closed-form initialisation).

Each test checks the oracle against something other than itself: an explicit
least-squares solve of eq. (13) over every entry of M, the minimum of the loss
under perturbation, cases with a known answer, and an independent enumeration of
the pairings of eq. (14) by permutations. A dropped S_b term, a transposed S, a
missing pseudo-inverse or a wrong head group fails one of them.
"""
import itertools

import numpy as np
import pytest

from oracle import convert_oracle as cv


def case(seed, T=9, D=5, d=3, h_q=4, h_k=2, rank=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, D))
    if rank is not None:                      # hidden states confined to a subspace
        X = X[:, :rank] @ rng.standard_normal((rank, D))
    W_Q = rng.standard_normal((D, h_q * d))
    W_K = rng.standard_normal((D, h_k * d))
    return X, W_Q, W_K


def lstsq_merge(X, W_Q, W_K, h_q, h_k, d, a, b):
    """Eq. (13) minimised by a generic least-squares solve: every logit entry
    Q^j[t] . (X M)[s] is linear in the entries M[x, c] with coefficient
    Q^j[t, c] * X[s, x]; the target is Q^j[t] . (X W_r)[s]."""
    T, D = X.shape
    rows, rhs = [], []
    for r in (a, b):
        W_r = W_K[:, r * d:(r + 1) * d]
        for j in cv.query_heads_of(r, h_q, h_k):
            Qj = X @ W_Q[:, j * d:(j + 1) * d]
            target = Qj @ (X @ W_r).T
            for t in range(T):
                for s in range(T):
                    rows.append(np.outer(X[s], Qj[t]).reshape(-1))   # index x * d + c
                    rhs.append(target[t, s])
    sol, *_ = np.linalg.lstsq(np.array(rows), np.array(rhs), rcond=None)
    return sol.reshape(D, d)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_closed_form_equals_least_squares(seed):
    h_q, h_k, d = 4, 2, 3
    X, W_Q, W_K = case(seed)
    t = cv.pair_table(X, W_Q, W_K, h_q, h_k, d)
    M = t.merged[(0, 1)]
    M_ls = lstsq_merge(X, W_Q, W_K, h_q, h_k, d, 0, 1)
    np.testing.assert_allclose(M, M_ls, rtol=0, atol=1e-9 * np.abs(M_ls).max())
    heads = [cv.query_heads_of(r, h_q, h_k) for r in range(2)]
    loss_ls = cv.pair_loss(X, W_Q, heads[0], heads[1], W_K[:, :d], W_K[:, d:], M_ls, d)
    assert abs(t.loss[0, 1] - loss_ls) <= 1e-9 * loss_ls


@pytest.mark.parametrize("rank", [None, 2])
def test_rank_deficient_closed_form_is_a_minimiser(rank):
    # no query uses the last head coordinate, so S_a + S_b is singular and the
    # minimiser is not unique (with rank=2 the hidden states also lie in a plane);
    # the pseudo-inverse form still reaches the least-squares minimum of eq. (13)
    h_q, h_k, d = 4, 2, 3
    X, W_Q, W_K = case(7, rank=rank)
    W_Q[:, d - 1::d] = 0.0
    t = cv.pair_table(X, W_Q, W_K, h_q, h_k, d)
    assert np.linalg.matrix_rank(cv.gram_of_queries(X, W_Q, [0, 1, 2, 3], d)) < d
    M_ls = lstsq_merge(X, W_Q, W_K, h_q, h_k, d, 0, 1)
    heads = [cv.query_heads_of(r, h_q, h_k) for r in range(2)]
    loss_ls = cv.pair_loss(X, W_Q, heads[0], heads[1], W_K[:, :d], W_K[:, d:], M_ls, d)
    assert abs(t.loss[0, 1] - loss_ls) <= 1e-8 * max(loss_ls, 1.0)


def test_loss_is_minimal_under_perturbation():
    h_q, h_k, d = 6, 2, 4
    X, W_Q, W_K = case(3, T=20, D=8, d=4, h_q=6, h_k=2)
    t = cv.pair_table(X, W_Q, W_K, h_q, h_k, d)
    M = t.merged[(0, 1)]
    heads = [cv.query_heads_of(r, h_q, h_k) for r in range(2)]
    rng = np.random.default_rng(0)
    for _ in range(5):
        E = rng.standard_normal(M.shape)
        for eps in (1e-3, 1e-1):
            l2 = cv.pair_loss(X, W_Q, heads[0], heads[1], W_K[:, :d], W_K[:, d:], M + eps * E, d)
            assert l2 > t.loss[0, 1]


def test_identical_heads_merge_exactly():
    # W_a == W_b: the merged projection is that projection and the loss is zero
    h_q, h_k, d = 4, 2, 3
    X, W_Q, W_K = case(4, T=12)
    W_K[:, d:] = W_K[:, :d]
    t = cv.pair_table(X, W_Q, W_K, h_q, h_k, d)
    np.testing.assert_allclose(t.merged[(0, 1)], W_K[:, :d], rtol=0, atol=1e-10)
    assert t.loss[0, 1] <= 1e-18 * np.abs(X).max() ** 4


def test_query_groups_are_contiguous():
    assert cv.query_heads_of(0, 32, 8) == [0, 1, 2, 3]
    assert cv.query_heads_of(7, 32, 8) == [28, 29, 30, 31]
    assert cv.query_heads_of(1, 12, 2) == list(range(6, 12))


def test_heads_of_the_other_group_do_not_count():
    # changing the query projection of a head outside groups a and b leaves L_ab
    h_q, h_k, d = 6, 3, 2
    X, W_Q, W_K = case(5, T=10, D=4, d=2, h_q=6, h_k=3)
    t1 = cv.pair_table(X, W_Q, W_K, h_q, h_k, d)
    W_Q2 = W_Q.copy()
    W_Q2[:, 4 * d:6 * d] *= 3.0                # query heads 4, 5 belong to key head 2
    t2 = cv.pair_table(X, W_Q2, W_K, h_q, h_k, d)
    assert t1.loss[0, 1] == t2.loss[0, 1]
    assert t1.loss[0, 2] != t2.loss[0, 2]


def permutation_minimum(w):
    """Eq. (14) read literally: every ordering sigma of the heads pairs
    (sigma_1, sigma_2), (sigma_3, sigma_4), ...; the least total over all orderings."""
    n = w.shape[0]
    best = np.inf
    for sigma in itertools.permutations(range(n)):
        best = min(best, sum(w[sigma[2 * i], sigma[2 * i + 1]] for i in range(n // 2)))
    return best


@pytest.mark.parametrize("n,seed", [(2, 0), (4, 1), (6, 2), (8, 3)])
def test_matching_equals_permutation_search(n, seed):
    rng = np.random.default_rng(seed)
    w = rng.random((n, n))
    w = w + w.T
    pairs, total = cv.min_weight_perfect_matching(w)
    assert abs(total - permutation_minimum(w)) <= 1e-12
    assert sorted(v for p in pairs for v in p) == list(range(n))
    assert abs(sum(w[a, b] for a, b in pairs) - total) <= 1e-12


def test_matching_count():
    # (n - 1)!! perfect matchings: 105 for the 8 key heads of Llama 3.2-1B
    assert sum(1 for _ in cv.perfect_matchings(list(range(8)))) == 105
    assert sum(1 for _ in cv.perfect_matchings(list(range(6)))) == 15


def test_conversion_pairs_near_identical_heads():
    # four teacher heads where 0 ~ 2 and 1 ~ 3: merging those pairs costs almost
    # nothing, every other pairing costs a lot
    h_q, h_k, d = 8, 4, 3
    X, W_Q, W_K = case(6, T=16, D=6, d=3, h_q=8, h_k=4)
    rng = np.random.default_rng(9)
    W_K[:, 2 * d:3 * d] = W_K[:, 0:d] + 1e-3 * rng.standard_normal((6, d))
    W_K[:, 3 * d:4 * d] = W_K[:, d:2 * d] + 1e-3 * rng.standard_normal((6, d))
    c = cv.convert(X, W_Q, W_K, h_q, h_k, d)
    assert c.pairs == [(0, 2), (1, 3)]
    assert c.W_K.shape == (6, 2 * d)
    np.testing.assert_allclose(c.W_K[:, :d], c.table.merged[(0, 2)])
    assert c.loss < 1e-2 * min(c.table.loss[0, 1], c.table.loss[0, 3])
