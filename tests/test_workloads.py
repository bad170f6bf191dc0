"""The seeded generators: determinism, shapes, dtype rounding, planted spikes."""
import numpy as np
import torch

from sparse_decode_attention_saga_amd import workloads as wl


def test_deterministic_and_seed_dependent():
    a = wl.generate(wl.TINY, seed=0)
    b = wl.generate(wl.TINY, seed=0)
    c = wl.generate(wl.TINY, seed=1)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v) and torch.equal(a.q, b.q)
    assert not torch.equal(a.k, c.k)


def test_shapes_dtype_and_exact_f64():
    w = wl.LLAMA_32K.with_(l_kv=2048)
    x = wl.generate(w, seed=0)
    assert x.q.shape == (1, 32, 64) and x.k.shape == (1, 2, 2048, 64) and x.v.shape == (1, 8, 2048, 64)
    assert x.k.dtype == torch.bfloat16
    q64, k64, v64 = x.f64()
    # bf16 values are exact in f64: round-tripping through bf16 changes nothing.
    assert np.array_equal(torch.from_numpy(k64).to(torch.bfloat16).to(torch.float64).numpy(), k64)


def test_planted_keys_score_about_three():
    x = wl.generate(wl.TINY, seed=0)
    q, K, _ = x.f64()
    A = (K[0, 0] @ q[0].T) / 8.0                      # [L, h_q] logits, d = 64
    n_planted = int(round(0.01 * 1024))
    top = np.sort(A.max(axis=1))[::-1][:n_planted]
    assert top.min() > 2.2 and abs(np.median(top) - 3.0) < 0.5
    # Background logits are about N(0, 1).
    assert 0.8 < np.std(A) < 1.3


def test_ragged_lengths_and_runs():
    w = wl.RAGGED_B8.with_(l_kv=4096, l_kv_min=1024)
    x = wl.generate(w, seed=3)
    assert x.l_kv.min() >= 1024 and x.l_kv.max() <= 4096 and x.l_max == int(x.l_kv.max())
    for b in range(8):
        L = int(x.l_kv[b])
        assert torch.count_nonzero(x.k[b, :, L:]) == 0 and torch.count_nonzero(x.v[b, :, L:]) == 0
    # planted runs: find rows with norm ~3 (planted) and check they come in 64-runs
    k = x.k[0, 0, : int(x.l_kv[0])].float()
    planted = (k.norm(dim=-1) < 4.0).nonzero().flatten().numpy()
    if planted.size:
        assert planted.size % 64 == 0
        starts = planted[::64]
        assert np.all(starts % 64 == 0)


def test_decode_stream_appends_and_drifts():
    w = wl.SWEEP.with_(l_kv=64)
    s = wl.DecodeStream(w, seed=0, l0=64, l_max=80)
    q0 = s.q.clone()
    s.append(3)
    s.drift()
    assert int(s.l_kv[0]) == 67
    assert torch.count_nonzero(s.k[0, :, 64:67]) > 0 and torch.count_nonzero(s.k[0, :, 67:]) == 0
    corr = torch.nn.functional.cosine_similarity(q0.float().flatten(), s.q.float().flatten(), dim=0)
    assert corr > 0.95
