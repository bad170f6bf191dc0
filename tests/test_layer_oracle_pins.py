"""Pins of the decode-layer oracle to facts that do not come from the oracle itself:
a library rounding routine, exact special cases of the products, and closed forms of
the whole layer on constructed inputs."""
import numpy as np
import torch

from oracle import layer_oracle as lo


def test_round_bf16_matches_torch_rounding_of_float32_values():
    rng = np.random.default_rng(0)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(10.0),
                          rng.uniform(-1e-3, 1e-3, 2000).astype(np.float32),
                          rng.uniform(1e3, 3e4, 2000).astype(np.float32)])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(lo.round_bf16(x32.astype(np.float64)), want)


def test_round_bf16_ties_go_to_even():
    u = 2.0 ** -7                                   # bf16 spacing in [1, 2)
    got = lo.round_bf16(np.array([1 + u / 2, 1 + 1.5 * u, -(1 + u / 2), 0.0, 255.5, 257.0, 1 + u / 2 + 1e-12]))
    assert got.tolist() == [1.0, 1 + 2 * u, -1.0, 0.0, 256.0, 256.0, 1 + u]


def test_linear_special_cases():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 8))
    perm = rng.permutation(8)
    P = np.eye(8)[perm]                             # row o picks input perm[o]
    assert np.array_equal(lo.linear(x, P), x[:, perm])
    a, b = rng.standard_normal(5), rng.standard_normal(8)
    np.testing.assert_allclose(lo.linear(x, np.outer(a, b)), np.outer(x @ b, a), rtol=1e-13, atol=1e-13)


def layer_inputs(B=2, D=None, h_q=4, h_k=1, h_v=2, d=8, l_max=10, lens=(6, 9), seed=0):
    """Caches of exact bf16 values, weights with bf16-exact entries, x one-hot per sequence."""
    rng = np.random.default_rng(seed)
    D = D or h_q * d
    K = lo.round_bf16(rng.standard_normal((B, h_k, l_max, d)))
    V = lo.round_bf16(rng.standard_normal((B, h_v, l_max, d)))
    for b in range(B):
        K[b, :, lens[b]:] = 0.0
        V[b, :, lens[b]:] = 0.0
    w_qkv = lo.round_bf16(rng.standard_normal(((h_q + h_k + h_v) * d, D)))
    w_o = lo.round_bf16(rng.standard_normal((D, h_q * d)))
    x = np.zeros((B, D))
    for b in range(B):
        x[b, b] = 1.0                              # projections = column b of each weight
    return x, w_qkv, w_o, K, V, np.asarray(lens)


def test_zero_query_keeps_every_row_and_averages_values_with_the_new_row():
    # q = 0: every logit is 0, the refreshed threshold keeps all l_kv + 1 rows (ties
    # kept), so the attention output is the mean of the value rows, new row included
    x, w_qkv, w_o, K, V, lens = layer_inputs()
    h_q, d = 4, 8
    w_qkv[: h_q * d] = 0.0                           # W_Q = 0
    r = lo.decode_layer(x, w_qkv, w_o, K, V, lens, h_q, "atopn", N=3, refresh_period=1, step=0)
    for b in range(2):
        L = lens[b]
        v_new = lo.round_bf16(w_qkv[(h_q + 1) * d:, b]).reshape(2, d)
        for j in range(h_q):
            vh = j * 2 // h_q
            want = (V[b, vh, :L].sum(axis=0) + v_new[vh]) / (L + 1)
            np.testing.assert_allclose(r.O[b, j], want, rtol=1e-12, atol=1e-12)
            assert r.attn.sel[b][j].tolist() == list(range(L + 1))
        np.testing.assert_allclose(r.y[b], w_o @ lo.round_bf16(r.O[b].reshape(-1)), rtol=1e-12)
    assert r.l_next.tolist() == [7, 10]


def test_dominant_new_key_selects_only_the_new_token():
    # the new key is a large multiple of every head's query: with N = 1 at a refresh
    # step only row l_kv[b] is kept, and head j outputs the new value row of v(j)
    x, w_qkv, w_o, K, V, lens = layer_inputs(h_q=4, h_k=1, h_v=4)
    h_q, d = 4, 8
    qrow = lo.round_bf16(np.abs(np.random.default_rng(5).standard_normal(d)) + 0.5)
    for b in range(2):
        for j in range(h_q):
            w_qkv[j * d:(j + 1) * d, b] = qrow
        w_qkv[h_q * d:(h_q + 1) * d, b] = 64.0 * qrow  # the new key
    r = lo.decode_layer(x, w_qkv, w_o, K, V, lens, h_q, "atopn", N=1, refresh_period=4, step=8)
    for b in range(2):
        v_new = lo.round_bf16(w_qkv[(h_q + 1) * d:, b]).reshape(4, d)
        for j in range(h_q):
            assert r.attn.sel[b][j].tolist() == [lens[b]]
            np.testing.assert_allclose(r.O[b, j], v_new[j], rtol=0, atol=0)
        np.testing.assert_allclose(r.K[b, 0, lens[b]], 64.0 * qrow, rtol=0, atol=0)


def test_dense_layer_over_an_empty_cache_returns_the_projected_new_value():
    # with nothing cached, the softmax has one entry: O_j = the new value row of v(j)
    x, w_qkv, w_o, K, V, _ = layer_inputs(lens=(0, 0))
    h_q, d = 4, 8
    r = lo.decode_layer(x, w_qkv, w_o, K, V, np.array([0, 0]), h_q, "dense")
    for b in range(2):
        v_new = lo.round_bf16(w_qkv[(h_q + 1) * d:, b]).reshape(2, d)
        want_o = np.stack([v_new[j * 2 // h_q] for j in range(h_q)])
        np.testing.assert_array_equal(r.O[b], want_o)
        np.testing.assert_allclose(r.y[b], w_o @ want_o.reshape(-1), rtol=1e-12)
    assert r.l_next.tolist() == [1, 1]


def test_full_cache_gets_no_new_row():
    x, w_qkv, w_o, K, V, _ = layer_inputs(lens=(10, 3))
    r = lo.decode_layer(x, w_qkv, w_o, K, V, np.array([10, 3]), 4, "dense")
    assert r.l_next.tolist() == [10, 4]
    np.testing.assert_array_equal(r.K[0], K[0])
    np.testing.assert_array_equal(r.V[0], V[0])
