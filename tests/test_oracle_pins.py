"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a library
attention routine, a brute-force pure-Python top-N, hand-built cases with a known
answer, invariants and the worked example of the explainer page. Together they
fail on a dropped scale, a sign error in the softmax, a wrong key/value head map,
a transposed operand, '>' instead of '>=', or a wrong refresh schedule.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import bytemodel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, B=2, h_q=8, h_k=2, h_v=4, d=16, L_max=40, lens=(40, 23), d_v=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, h_q, d))
    K = rng.standard_normal((B, h_k, L_max, d))
    V = rng.standard_normal((B, h_v, L_max, d if d_v is None else d_v))
    return q, K, V, np.array(lens[:B])


def sdpa_row(q_j, K_rows, V_rows, mask=None):
    """torch's attention on one query row (float64, CPU); default scale 1/sqrt(d)."""
    qt = torch.from_numpy(q_j)[None, None, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K_rows))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(V_rows))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0, 0, 0].numpy()


def brute_topn(q_j, K_rows, N):
    """Pure-Python: logits by explicit loops, then the N best indices by a full sort."""
    d = len(q_j)
    s = 1.0 / math.sqrt(d)
    scores = [sum(float(q_j[c]) * float(K_rows[i][c]) for c in range(d)) * s
              for i in range(len(K_rows))]
    order = sorted(range(len(scores)), key=lambda i: -scores[i])
    return sorted(order[:N]), scores


# --- dense limit (N >= l_kv) and GQA reduce to library attention ----------------

@pytest.mark.parametrize("h_k,h_v", [(2, 4), (1, 8), (4, 4), (8, 2)])
def test_dense_limit_equals_library_attention(h_k, h_v):
    q, K, V, lens = rand_case(1, h_q=8, h_k=h_k, h_v=h_v)
    r = orc.saga_decode_step(q, K, V, lens, N=10 ** 6, refresh_period=1, step=0)
    for b in range(q.shape[0]):
        L = lens[b]
        for j in range(8):
            g, v = j * h_k // 8, j * h_v // 8
            ref = sdpa_row(q[b, j], K[b, g, :L], V[b, v, :L])
            np.testing.assert_allclose(r.O[b, j], ref, rtol=0, atol=1e-12)
            assert r.sel[b][j].tolist() == list(range(L))
            assert r.tau[b, j] == -np.inf


@pytest.mark.parametrize("scale", [0.05, 1.0, 2.5])
def test_given_scale_equals_library_attention(scale):
    # eq. (2) with a logit scale other than 1/sqrt(d): torch's attention with the same scale
    q, K, V, lens = rand_case(2, h_q=4, h_k=1, h_v=2)
    r = orc.saga_decode_step(q, K, V, lens, N=10 ** 6, refresh_period=1, step=0, scale=scale)
    d = orc.dense_gqa(q, K, V, lens, scale=scale)
    for b in range(q.shape[0]):
        L = lens[b]
        for j in range(4):
            qt = torch.from_numpy(q[b, j])[None, None, None, :]
            kt = torch.from_numpy(np.ascontiguousarray(K[b, 0, :L]))[None, None]
            vt = torch.from_numpy(np.ascontiguousarray(V[b, j * 2 // 4, :L]))[None, None]
            ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()
            np.testing.assert_allclose(r.O[b, j], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(d[b, j], ref, rtol=0, atol=1e-12)
    # and the selection is made on the scaled logits: with N = 1 the largest entry is
    # kept whatever the (positive) scale
    r1 = orc.saga_decode_step(q, K, V, lens, N=1, refresh_period=1, step=0, scale=scale)
    for b in range(q.shape[0]):
        L = lens[b]
        for j in range(4):
            a = K[b, 0, :L] @ q[b, j]
            assert r1.sel[b][j].tolist() == [int(np.argmax(a))]
            assert abs(r1.tau[b, j] - scale * a.max()) <= 1e-12 * abs(scale * a.max())


def test_equal_heads_is_grouped_query_attention():
    # h_k == h_v: the library's own grouped-query attention (enable_gqa) fixes the
    # head grouping independently of the oracle's head maps.
    q, K, V, _ = rand_case(2, B=2, h_q=8, h_k=2, h_v=2, L_max=30, lens=(30, 30))
    lens = np.array([30, 30])
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(K), torch.from_numpy(V),
        enable_gqa=True)[:, :, 0].numpy()
    sparse = orc.saga_decode_step(q, K, V, lens, N=30, refresh_period=1, step=0)
    np.testing.assert_allclose(sparse.O, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.dense_gqa(q, K, V, lens), ref, rtol=0, atol=1e-12)


def test_dense_gqa_ragged_lengths():
    q, K, V, lens = rand_case(3, h_k=4, h_v=4)
    O = orc.dense_gqa(q, K, V, lens)
    for b in range(2):
        for j in range(8):
            ref = sdpa_row(q[b, j], K[b, j // 2, :lens[b]], V[b, j // 2, :lens[b]])
            np.testing.assert_allclose(O[b, j], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("h_k,h_v", [(1, 4), (2, 8), (1, 12)])
def test_dense_saga_full_attention(h_k, h_v):
    # h_k < h_v (SAGA, full attention): torch's attention with the key cache and the
    # value cache each expanded to the query heads by its own group size
    h_q = 12 if h_v == 12 else 8
    q, K, V, lens = rand_case(4 + h_v, h_q=h_q, h_k=h_k, h_v=h_v)
    O = orc.dense_gqa(q, K, V, lens)
    Kx = torch.from_numpy(K).repeat_interleave(h_q // h_k, dim=1)
    Vx = torch.from_numpy(V).repeat_interleave(h_q // h_v, dim=1)
    for b in range(q.shape[0]):
        L = int(lens[b])
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[b])[:, None, :], Kx[b, :, :L], Vx[b, :, :L])[:, 0]
        np.testing.assert_allclose(O[b], ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("d,d_v", [(8, 16), (16, 32), (32, 8)])
def test_value_dim_differs_from_key_dim(d, d_v):
    # a key head dimension below (or above) the value head dimension: torch's
    # attention takes value rows of their own width and scales by 1/sqrt(d) of q, k
    q, K, V, lens = rand_case(40 + d, h_q=8, h_k=2, h_v=4, d=d, d_v=d_v)
    dense = orc.dense_gqa(q, K, V, lens)
    full = orc.saga_decode_step(q, K, V, lens, N=10 ** 6, refresh_period=1, step=0)
    Kx = torch.from_numpy(K).repeat_interleave(4, dim=1)
    Vx = torch.from_numpy(V).repeat_interleave(2, dim=1)
    for b in range(q.shape[0]):
        L = int(lens[b])
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[b])[:, None, :], Kx[b, :, :L], Vx[b, :, :L])[:, 0]
        np.testing.assert_allclose(dense[b], ref.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(full.O[b], ref.numpy(), rtol=0, atol=1e-12)
    # and the top-N selection is that of the logits alone: with N = 3 the masked
    # library attention over each row's three best keys
    top = orc.saga_decode_step(q, K, V, lens, N=3, refresh_period=1, step=0)
    for b in range(q.shape[0]):
        L = int(lens[b])
        for j in range(8):
            want, _ = brute_topn(q[b, j], K[b, j // 4, :L], 3)
            assert top.sel[b][j].tolist() == want
            mask = np.zeros(L, bool)
            mask[want] = True
            ref = sdpa_row(q[b, j], K[b, j // 4, :L], V[b, j // 2, :L], mask)
            assert top.O[b, j].shape == (d_v,)
            np.testing.assert_allclose(top.O[b, j], ref, rtol=0, atol=1e-12)


# --- refresh step = exact top-N (eq. 6-7) ---------------------------------------

@pytest.mark.parametrize("N", [1, 2, 7, 22, 23])
def test_refresh_equals_bruteforce_topn(N):
    q, K, V, lens = rand_case(4, h_q=4, h_k=1, h_v=2, d=8, L_max=30, lens=(30, 23))
    r = orc.saga_decode_step(q, K, V, lens, N=N, refresh_period=1, step=0)
    for b in range(2):
        L = lens[b]
        for j in range(4):
            want, scores = brute_topn(q[b, j], K[b, 0, :L], N)
            assert r.sel[b][j].tolist() == want
            mask = np.zeros(L, bool)
            mask[want] = True
            ref = sdpa_row(q[b, j], K[b, 0, :L], V[b, j // 2, :L], mask)
            np.testing.assert_allclose(r.O[b, j], ref, rtol=0, atol=1e-12)
            if N < L:
                assert math.isclose(r.tau[b, j], sorted(scores)[::-1][N - 1], rel_tol=1e-12)
                assert len(want) == N


# Key head of each of 8 query heads, written out per key-head count (contiguous
# groups of h_q / h_k query heads, as in grouped-query attention).
KEY_HEAD_OF_8 = {1: [0] * 8, 2: [0, 0, 0, 0, 1, 1, 1, 1], 4: [0, 0, 1, 1, 2, 2, 3, 3]}


@pytest.mark.parametrize("h_k", [1, 2, 4])
@pytest.mark.parametrize("scale", [None, 0.3])
def test_refresh_threshold_equals_bruteforce_sort(h_k, scale):
    # The exact threshold of a refresh step (section "Top-N Attention", eq. (6); the
    # Atop-N threshold is the N-th largest logit of the row): pure-Python logits of
    # each row against its key head, then the N-th entry of a full descending sort,
    # counting repeats. Rows cover an empty sequence (no threshold: NaN), N >= l_kv
    # (-inf: everything kept), N = l_kv - 1, and keys repeated to force ties.
    h_q, d, L_max = 8, 6, 24
    rng = np.random.default_rng(40 + h_k)
    q = rng.standard_normal((4, h_q, d))
    K = rng.standard_normal((4, h_k, L_max, d))
    K[:, :, 5] = K[:, :, 2]           # repeated keys: tied logits around the threshold
    K[:, :, 9] = K[:, :, 2]
    lens = np.array([24, 0, 7, 13])
    s = (1.0 / math.sqrt(d)) if scale is None else scale
    for N in (1, 3, 6, 7, 12, 30):
        got = orc.refresh_threshold(q, K, lens, N, scale=scale)
        for b in range(4):
            L = int(lens[b])
            for j in range(h_q):
                g = KEY_HEAD_OF_8[h_k][j]
                if L == 0:
                    assert math.isnan(got[b, j])
                    continue
                scores = [sum(float(q[b, j, c]) * float(K[b, g, i, c]) for c in range(d)) * s for i in range(L)]
                want = -math.inf if N >= L else sorted(scores, reverse=True)[N - 1]
                if want == -math.inf:
                    assert got[b, j] == -math.inf, (b, j, N)
                else:
                    assert math.isclose(got[b, j], want, rel_tol=1e-12, abs_tol=1e-14), (b, j, N)
    # the tie: with N = 2 or 3 the three repeated keys of a row whose repeated key is
    # the largest give one threshold value, that key's logit
    Kt = K.copy()
    Kt[0, :, 2] = 50.0 * np.sign(q[0, 0]) / math.sqrt(d)   # largest logit of head 0's key head
    Kt[0, :, 5] = Kt[0, :, 2]
    Kt[0, :, 9] = Kt[0, :, 2]
    top = sum(float(q[0, 0, c]) * float(Kt[0, 0, 2, c]) for c in range(d)) * s
    for N in (1, 2, 3):
        assert math.isclose(orc.refresh_threshold(q, Kt, lens, N, scale=scale)[0, 0], top, rel_tol=1e-12)


def test_nth_largest_matches_partition_with_repeats():
    rng = np.random.default_rng(5)
    for _ in range(200):
        L = int(rng.integers(1, 60))
        a = rng.integers(-4, 5, size=L).astype(np.float64) * 0.5  # many repeats, +-0
        N = int(rng.integers(1, L + 3))
        want = -np.inf if N >= L else np.partition(a, L - N)[L - N]
        assert orc.nth_largest(a, N) == want


# --- threshold semantics: >=, ties kept, largest not smallest -------------------

def test_ties_at_threshold_are_all_kept():
    # d=4, q = e0, so logit_i = K[i,0] / 2; five keys tie at the 3rd-largest value.
    q = np.zeros((1, 1, 4)); q[0, 0, 0] = 1.0
    col = np.array([10., 8., 6., 6., 6., 4., 2.])
    K = np.zeros((1, 1, 7, 4)); K[0, 0, :, 0] = col
    V = np.arange(7 * 4, dtype=np.float64).reshape(1, 1, 7, 4)
    lens = np.array([7])
    expect = {1: [0], 2: [0, 1], 3: [0, 1, 2, 3, 4], 5: [0, 1, 2, 3, 4], 6: [0, 1, 2, 3, 4, 5], 7: list(range(7))}
    for N, idx in expect.items():
        r = orc.saga_decode_step(q, K, V, lens, N=N, refresh_period=1, step=0)
        assert r.sel[0][0].tolist() == idx, N
        if N < 7:
            assert r.tau[0, 0] == col[N - 1] / 2


def test_identical_keys_keep_everything_and_average_values():
    # All logits equal: the N-th largest equals every logit, all tie and are kept,
    # and the softmax is uniform, so O is the mean of the value rows.
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, 8))
    K = np.repeat(rng.standard_normal((1, 1, 1, 8)), 50, axis=2)
    V = rng.standard_normal((1, 2, 50, 8))
    r = orc.saga_decode_step(q, K, V, np.array([50]), N=5, refresh_period=1, step=0)
    for j in range(2):
        assert r.sel[0][j].size == 50
        np.testing.assert_allclose(r.O[0, j], V[0, j].mean(axis=0), rtol=0, atol=1e-12)


def test_head_maps_and_largest_entry():
    # h_q=6, h_k=2, h_v=3. Key head g holds one huge key at position p[g]; with
    # N=1 query head j must pick p[g(j)] and return value row V[v(j), p[g(j)]].
    h_q, h_k, h_v, d, L = 6, 2, 3, 8, 20
    rng = np.random.default_rng(7)
    p = [3, 11]
    q = np.zeros((1, h_q, d)); q[0, :, 0] = 1.0
    K = 0.01 * rng.standard_normal((1, h_k, L, d))
    K[0, 0, p[0], 0] = 10.0
    K[0, 1, p[1], 0] = 10.0
    K[0, 0, p[1], 0] = -10.0          # the other head's spike is a minimum here
    V = np.zeros((1, h_v, L, d))
    for h in range(h_v):
        for i in range(L):
            V[0, h, i, 0], V[0, h, i, 1] = h, i
    r = orc.saga_decode_step(q, K, V, np.array([L]), N=1, refresh_period=1, step=0)
    g_of = [0, 0, 0, 1, 1, 1]
    v_of = [0, 0, 1, 1, 2, 2]
    for j in range(h_q):
        assert r.sel[0][j].tolist() == [p[g_of[j]]]
        assert r.O[0, j, 0] == v_of[j] and r.O[0, j, 1] == p[g_of[j]]


# --- invariants ------------------------------------------------------------------

def test_probabilities_sum_to_one_and_output_is_convex():
    q, K, V, lens = rand_case(8, d=32, L_max=200, lens=(200, 150))
    for N in (1, 5, 64):
        r = orc.saga_decode_step(q, K, V, lens, N=N, refresh_period=1, step=0)
        assert np.all(np.abs(r.sum_p - 1.0) <= 1e-12)
        for b in range(2):
            for j in range(8):
                rows = V[b, j * 4 // 8, r.sel[b][j]]
                assert np.all(r.O[b, j] >= rows.min(axis=0) - 1e-12)
                assert np.all(r.O[b, j] <= rows.max(axis=0) + 1e-12)


def test_key_permutation_permutes_selection_only():
    q, K, V, lens = rand_case(9, B=1, lens=(40,))
    perm = np.random.default_rng(10).permutation(40)
    r1 = orc.saga_decode_step(q, K, V, lens, N=6, refresh_period=1, step=0)
    r2 = orc.saga_decode_step(q, K[:, :, perm], V[:, :, perm], lens, N=6, refresh_period=1, step=0)
    np.testing.assert_allclose(r1.O, r2.O, rtol=0, atol=1e-12)
    for j in range(8):
        assert sorted(perm[r2.sel[0][j]].tolist()) == r1.sel[0][j].tolist()


def test_empty_sequence():
    q, K, V, _ = rand_case(11)
    tau_in = np.full((2, 8), 0.25)
    r = orc.saga_decode_step(q, K, V, np.array([0, 23]), N=4, refresh_period=4, step=1, tau_in=tau_in)
    assert np.all(r.O[0] == 0) and np.all(r.tau[0] == 0.25)
    assert all(s.size == 0 for s in r.sel[0])


# --- periodic refresh and stale thresholds ---------------------------------------

def test_stale_threshold_reused_between_refreshes():
    # Frozen q and K: stale steps keep exactly the refresh step's selection; the
    # exact threshold is recomputed at t = 0 and t = 3 only (period n = 3).
    q, K, V, lens = rand_case(12, B=1, lens=(40,))
    tau = None
    sels = []
    for t in range(6):
        r = orc.saga_decode_step(q, K, V, lens, N=5, refresh_period=3, step=t, tau_in=tau)
        assert bool(r.refreshed.all()) == (t % 3 == 0)
        assert not r.fallback.any()
        sels.append([s.tolist() for s in r.sel[0]])
        tau = r.tau
    assert all(s == sels[0] for s in sels)


def test_appended_keys_compare_against_stale_threshold():
    q, K, V, lens = rand_case(13, B=1, h_q=2, h_k=1, h_v=1, d=8, L_max=40, lens=(30,))
    r0 = orc.saga_decode_step(q, K, V, lens, N=4, refresh_period=8, step=0)
    K2 = K.copy()
    # Position 30 gets a key far above head 0's threshold, position 31 far below.
    K2[0, 0, 30] = 20.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    K2[0, 0, 31] = -20.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    r1 = orc.saga_decode_step(q, K2, V, np.array([32]), N=4, refresh_period=8, step=1, tau_in=r0.tau)
    assert r1.tau[0, 0] == r0.tau[0, 0]
    assert r1.sel[0][0].tolist() == sorted(r0.sel[0][0].tolist() + [30])
    assert 31 not in r1.sel[0][1].tolist() or r1.logits[0][1][31] >= r0.tau[0, 1]
    # The next refresh (t = 8) recomputes the 4-th largest of the grown row: 5 -> 4 kept.
    r8 = orc.saga_decode_step(q, K2, V, np.array([32]), N=4, refresh_period=8, step=8, tau_in=r1.tau)
    assert r8.sel[0][0].size == 4 and 30 in r8.sel[0][0].tolist()


def test_empty_stale_selection_forces_refresh():
    q, K, V, lens = rand_case(14)
    tau_in = np.full((2, 8), np.inf)
    tau_in[1, 3] = -np.inf            # this row keeps everything under its stale threshold
    r = orc.saga_decode_step(q, K, V, lens, N=3, refresh_period=5, step=2, tau_in=tau_in)
    exact = orc.saga_decode_step(q, K, V, lens, N=3, refresh_period=1, step=0)
    for b in range(2):
        for j in range(8):
            if (b, j) == (1, 3):
                assert not r.fallback[b, j] and r.sel[b][j].size == lens[b]
                continue
            assert r.fallback[b, j]
            assert r.sel[b][j].tolist() == exact.sel[b][j].tolist()
            np.testing.assert_allclose(r.O[b, j], exact.O[b, j], rtol=0, atol=0)


# --- the explainer's worked example pins the byte model --------------------------

def test_explainer_vector_read_table():
    rows, ratios = {}, {}
    with open(os.path.join(GOLDEN, "explainer_vector_reads.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "ratio":
                ratios[parts[1]] = float(parts[2])
            else:
                rows[parts[0]] = parts[1:]
    for name, (h_q, h_k, h_v, L, N, kr, vr, tot) in rows.items():
        got = bytemodel.vector_reads(int(h_q), int(h_k), int(h_v), int(L), None if N == "-" else int(N))
        assert got == (int(kr), int(vr), int(tot)), name
    d = dict((k, int(v[-1])) for k, v in rows.items())
    kg = int(rows["gqa_topn"][5])
    assert round(kg / d["gqa_topn"], 2) == ratios["keys_share_gqa_topn"]
    assert round(d["gqa_topn"] / d["saga_topn"], 1) == ratios["gqa_topn_over_saga"]
    assert round(d["dense_gqa"] / d["saga_topn"], 1) == ratios["dense_over_saga"]
    # bytes: keys stream h_k * l_kv * d * s; dense streams keys and values
    assert bytemodel.key_bytes(4, 64, [131072], 2) == 524288 * 64 * 2
    assert bytemodel.dense_bytes(8, 64, [131072], 2) == 2097152 * 64 * 2
