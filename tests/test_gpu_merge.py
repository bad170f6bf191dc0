"""The GQA-to-SAGA key-head merge on the GPU against the CPU oracle (needs an MI355X).

Tolerances (derived from the arithmetic of the GPU path): the inputs are bf16 and
exact in both paths; the GPU forms queries, keys and their Gram matrices with fp32
accumulation (sums of up to D and g*T products of random-sign terms, relative
error about 2^-24 * sqrt(terms) <= 1e-6 for the sizes here), then works in fp64:
  * a pair's loss L_ab agrees within 1e-5 L_ab + 1e-7 E_ab, where E_ab is the logit
    energy of the two heads (sum over their query heads of ||Q^j K_r^T||_F^2): the
    loss is a residual of that energy, so its absolute error scales with E_ab;
  * merged projections agree normwise within 1e-5 of max |M|;
  * the pairing is the oracle's unless another pairing's total lies within the
    loss tolerance of the optimum (then either is correct: both are checked to be
    within it).
"""
import numpy as np
import pytest
import torch

from oracle import convert_oracle as cv
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[merge] {msg}", flush=True)


def energy(X, W_Q, W_K, h_q, h_k, d, r):
    K = X @ cv.head_block(W_K, r, d)
    return sum(float(np.linalg.norm((X @ cv.head_block(W_Q, j, d)) @ K.T) ** 2)
               for j in cv.query_heads_of(r, h_q, h_k))


def check_merge(T, D, h_q, h_k, d, seed, twins=()):
    inp = wl.merge_inputs(T, D, h_q, h_k, d, seed=seed, twins=twins)
    X = inp.x.double().numpy()
    W_Q = inp.w_q.double().numpy().T      # the pages' orientation [D, h d]
    W_K = inp.w_k.double().numpy().T
    ref = cv.convert(X, W_Q, W_K, h_q, h_k, d)
    x, wq, wk = inp.x.to(DEV), inp.w_q.to(DEV), inp.w_k.to(DEV)
    loss, ws = api.merge_losses(x, wq, wk, h_q=h_q, h_k=h_k)
    got = loss.double().cpu().numpy()
    E = [energy(X, W_Q, W_K, h_q, h_k, d, r) for r in range(h_k)]
    worst = 0.0
    for a in range(h_k):
        assert got[a, a] == 0.0
        for b in range(a + 1, h_k):
            want = ref.table.loss[a, b]
            assert got[a, b] == got[b, a]
            tol = 1e-5 * want + 1e-7 * (E[a] + E[b])
            err = abs(got[a, b] - want)
            worst = max(worst, err / tol)
            assert err <= tol, (a, b, got[a, b], want)
    # the pairing: the oracle's, or one whose oracle total is as good within tolerance
    partner, total = api.min_weight_pairing(loss.cpu())
    pairs = sorted((a, b) for a, b in enumerate(partner) if a < b)
    tol_total = sum(1e-5 * ref.table.loss[a, b] + 1e-7 * (E[a] + E[b]) for a, b in ref.pairs)
    if pairs != ref.pairs:
        alt = sum(ref.table.loss[a, b] for a, b in pairs)
        assert alt - ref.loss <= 2 * tol_total, (pairs, ref.pairs)
    # merged projections of the oracle's pairing
    part = [0] * h_k
    for a, b in ref.pairs:
        part[a], part[b] = b, a
    out = api.merge_keys(x, wq, wk, part, h_q=h_q, h_k=h_k, workspace=ws)
    torch.cuda.synchronize()
    M = out.double().cpu().numpy().T      # [D, h_k/2 d]
    scale = np.abs(ref.W_K).max()
    merr = np.abs(M - ref.W_K).max() / scale
    say(f"T={T} D={D} h_q={h_q} h_k={h_k} d={d}: loss err/tol {worst:.3f}, merged rel err {merr:.2e}, "
        f"pairs {pairs} (oracle {ref.pairs})")
    assert merr <= 1e-5
    return pairs, ref


CASES = [
    # T, D, h_q, h_k, d
    (300, 256, 8, 4, 64),        # ragged token chunks and row tiles
    (100, 512, 8, 4, 128),
    (77, 96, 4, 2, 64),          # fewer tokens than one chunk
    (513, 1024, 16, 8, 64),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_merge_small(case):
    T, D, h_q, h_k, d = CASES[case]
    say(f"case {case}: {CASES[case]}")
    check_merge(T, D, h_q, h_k, d, seed=case)


def test_merge_planted_pairs():
    # heads (0, 5), (1, 2), (3, 7), (4, 6) are near-copies: the planted pairing wins
    twins = [(0, 5), (1, 2), (3, 7), (4, 6)]
    pairs, ref = check_merge(400, 512, 16, 8, 64, seed=10, twins=twins)
    assert pairs == sorted(twins) == ref.pairs


@pytest.mark.parametrize("name,T,D,h_q,h_k,d", [
    ("llama3.2-1b-shape", 512, 2048, 32, 8, 64),
    ("qwen2.5-1.5b-shape", 512, 1536, 12, 2, 128),
])
def test_merge_model_shapes(name, T, D, h_q, h_k, d):
    say(f"{name}: T={T}")
    check_merge(T, D, h_q, h_k, d, seed=20)


def test_rank_deficient_gram():
    # 12 calibration tokens and 4 query heads: S_a + S_b has rank at most 48 < d = 64,
    # the pseudo-inverse cut applies, and loss and merge are still the oracle's
    inp = wl.merge_inputs(12, 256, 4, 2, 64, seed=30)
    X, W_Q = inp.x.double().numpy(), inp.w_q.double().numpy().T
    S = sum(cv.gram_of_queries(X, W_Q, cv.query_heads_of(r, 4, 2), 64) for r in range(2))
    assert np.linalg.matrix_rank(S) == 48
    check_merge(12, 256, 4, 2, 64, seed=30)


def test_merge_twelve_heads():
    # 66 pairs, 10395 pairings
    check_merge(256, 512, 24, 12, 64, seed=40)


def test_merge_one_token():
    # one calibration token: each S_r has rank at most h_q / h_k, the sum of two at
    # most 4 < d, so every pair takes the eigendecomposition path with the cut
    check_merge(1, 256, 8, 4, 64, seed=41)


def test_merge_d128_four_heads_planted():
    twins = [(0, 3), (1, 2)]
    pairs, ref = check_merge(300, 768, 8, 4, 128, seed=42, twins=twins)
    assert pairs == sorted(twins)


def test_many_calibration_tokens_scale_the_losses():
    # past 16384 calibration tokens the partial Grams take longer token chunks. A
    # property that holds at any size: repeating every calibration token once
    # doubles the queries and keys, so every logit matrix appears four times, every
    # loss of eq. (13) is 4x the loss of the original tokens, and the merged
    # projections of eq. (15) (a ratio of Grams) are unchanged.
    T, D, h_q, h_k, d = 9000, 256, 8, 4, 64
    inp = wl.merge_inputs(T, D, h_q, h_k, d, seed=7)
    x = inp.x.to(DEV)
    x2 = torch.cat([x, x], dim=0)          # 18000 tokens
    wq, wk = inp.w_q.to(DEV), inp.w_k.to(DEV)
    say(f"T={T} and its doubled set {2 * T}")
    l1, ws1 = api.merge_losses(x, wq, wk, h_q=h_q, h_k=h_k)
    l2, ws2 = api.merge_losses(x2, wq, wk, h_q=h_q, h_k=h_k)
    a, b = l1.double().cpu().numpy(), l2.double().cpu().numpy()
    off = ~np.eye(h_k, dtype=bool)
    assert np.all(np.abs(b[off] - 4 * a[off]) <= 1e-4 * 4 * a[off])
    partner = list(api.min_weight_pairing(l1.cpu())[0])
    assert list(api.min_weight_pairing(l2.cpu())[0]) == partner
    m1 = api.merge_keys(x, wq, wk, partner, h_q=h_q, h_k=h_k, workspace=ws1)
    m2 = api.merge_keys(x2, wq, wk, partner, h_q=h_q, h_k=h_k, workspace=ws2)
    torch.cuda.synchronize()
    m1, m2 = m1.double().cpu().numpy(), m2.double().cpu().numpy()
    assert np.abs(m2 - m1).max() <= 1e-5 * np.abs(m1).max()
