"""Key heads of a smaller dimension than the value heads (d_k < d_v): the HIP path
against the CPU oracle on identical seeded inputs (needs an MI355X).

The pages compare fewer key heads with key heads of a reduced dimension (section
"Training from Scratch", the Sigma-style variant with (h_k, d_k) = (2, 32)); the
library builds (d_k, d_v) = (32, 64) for fp32 and bf16 and (64, 128) for bf16.
Logits use d_k (scale 1/sqrt(d_k)), outputs have d_v columns. Tolerances are those
of the other parity tests (tests/parity.py).
"""
import numpy as np
import pytest
import torch

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import GpuCase, compare
from tests.test_gpu_paged import PagedCase, same_selection

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[value-dim] {msg}", flush=True)


def small(B, h_q, h_k, h_v, d, d_v, lens, dtype, seed, l_max=None, plant=0.01):
    w = wl.Workload("small-dv", 290 + seed, batch=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, d_v=d_v, l_kv=max(lens),
                    N=1, refresh_period=1, dtype=dtype, plant_frac=plant)
    return wl.generate(w, seed=seed, lengths=lens, l_max=l_max or max(max(lens), 1))


def oracle_step(x, N, n, step, tau_in=None):
    q64, k64, v64 = x.f64()
    return orc.saga_decode_step(q64, k64, v64, x.l_kv, N, n, step, tau_in=tau_in)


CASES = [
    # B, h_q, h_k, h_v, d_k, d_v, lens, dtype, N
    (2, 8, 2, 4, 32, 64, [1000, 37], "f32", 16),
    (1, 4, 1, 4, 32, 64, [3001], "f32", 64),
    (2, 32, 4, 8, 32, 64, [5000, 513], "bf16", 32),
    (3, 12, 2, 4, 64, 128, [513, 1, 2000], "bf16", 32),
    (1, 12, 2, 4, 64, 128, [7000], "bf16", 200),
    (2, 16, 1, 16, 32, 64, [900, 0], "bf16", 8),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_reduced_key_dim_refresh_stale_forced(case):
    B, h_q, h_k, h_v, dk, dv, lens, dtype, N = CASES[case]
    say(f"case {case}: {CASES[case]}")
    x = small(B, h_q, h_k, h_v, dk, dv, lens, dtype, seed=case, l_max=max(lens) + 5)
    assert x.k.shape[3] == dk and x.v.shape[3] == dv
    g = GpuCase(x, N)
    got = g.step(4, 0)
    ref = oracle_step(x, N, 4, 0)
    assert got["O"].shape == (B, h_q, dv)
    compare(got, ref, x, dtype, check_tau=True)
    got1 = g.step(4, 1)
    compare(got1, oracle_step(x, N, 4, 1, tau_in=ref.tau), x, dtype, check_tau=False)
    assert np.array_equal(got1["count"], got["count"])
    # a stale threshold that keeps nothing: the forced exact refresh of every row
    tau_inf = np.full((B, h_q), np.inf, np.float32)
    got2 = g.step(4, 2, tau_in=tau_inf)
    ref2 = oracle_step(x, N, 4, 2, tau_in=tau_inf.astype(np.float64))
    compare(got2, ref2, x, dtype, check_tau=True)
    live = np.asarray(lens) > 0
    assert np.all(got2["flags"][live] == 3)


def test_reduced_key_dim_wide_chunks():
    # 16 sequences: the launch takes chunks of 512 keys (8 tiles per wave)
    lens = [16384, 1, 9000, 16383, 256, 511, 12000, 16384, 700, 16000, 3, 8192, 8193, 15000, 4097, 16384]
    x = small(16, 12, 2, 4, 64, 128, lens, "bf16", seed=20)
    say("chunks of 512 keys, (d_k, d_v) = (64, 128), B=16")
    g = GpuCase(x, 64, sel_cap=256)
    got = g.step(4, 0)
    ref = oracle_step(x, 64, 4, 0)
    compare(got, ref, x, "bf16", check_tau=True)
    got1 = g.step(4, 1)
    compare(got1, oracle_step(x, 64, 4, 1, tau_in=ref.tau), x, "bf16", check_tau=False)


@pytest.mark.parametrize("name", ["llama3.2-1b-shape-sigma-keys-l32k", "qwen2.5-1.5b-shape-sigma-keys-l128k"])
def test_sigma_keys_workload_full_size(name):
    w = wl.WORKLOADS[name]
    x = wl.generate(w, seed=0)
    say(f"{name}: refresh step then a stale step")
    g = GpuCase(x, w.N)
    got = g.step(w.refresh_period, 0)
    ref = oracle_step(x, w.N, w.refresh_period, 0)
    bands = compare(got, ref, x, w.dtype, check_tau=True)
    assert bands <= max(1, w.h_q // 8)
    got1 = g.step(w.refresh_period, 5)
    compare(got1, oracle_step(x, w.N, w.refresh_period, 5, tau_in=ref.tau), x, w.dtype, check_tau=False)


def test_reduced_key_dim_stages_and_threshold():
    x = small(1, 12, 2, 4, 64, 128, [6000], "bf16", seed=21)
    g = GpuCase(x, 64)
    g.step(8, 0)
    ref = g.step(8, 1)
    tau = g.tau.clone()
    out = torch.empty_like(g.out)
    api.qk_select(g.q, g.k, g.l_kv, tau, max_l_kv=g.max_l_kv, workspace=g.ws, d_v=128)
    api.sparse_gather(g.q, g.k, g.v, g.l_kv, tau, N=64, max_l_kv=g.max_l_kv, out=out, workspace=g.ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.double().cpu().numpy(), ref["O"], rtol=0, atol=1e-5 * np.abs(ref["O"]).max())
    q64, k64, _ = x.f64()
    for N in (1, 100, 6000):
        api.refresh_threshold(g.q, g.k, g.l_kv, g.tau, N=N, max_l_kv=g.max_l_kv, workspace=g.ws, d_v=128)
        torch.cuda.synchronize()
        got = g.tau.double().cpu().numpy()
        want = orc.refresh_threshold(q64, k64, x.l_kv, N)
        fin = np.isfinite(want)
        assert np.all(got[~fin] == want[~fin])
        assert np.all(np.abs(got[fin] - want[fin]) <= 1e-5 * np.abs(want[fin])), N


PAGED = [
    # B, h_q, h_k, h_v, d_k, d_v, lens, dtype, N, page_tokens
    (2, 12, 2, 4, 64, 128, [3000, 700], "bf16", 32, 64),
    (1, 8, 2, 4, 32, 64, [2500], "f32", 16, 16),
]


@pytest.mark.parametrize("case", range(len(PAGED)))
def test_reduced_key_dim_paged(case):
    B, h_q, h_k, h_v, dk, dv, lens, dtype, N, pt = PAGED[case]
    say(f"paged case {case}: {PAGED[case]}")
    x = small(B, h_q, h_k, h_v, dk, dv, lens, dtype, seed=30 + case)
    max_l_kv = x.k.shape[2]
    cap = min(max_l_kv, 4 * N)
    c = GpuCase(x, N, sel_cap=cap)
    p = PagedCase(x, N, pt, -1, seed=case, sel_cap=cap, max_l_kv=max_l_kv)
    for step in (0, 1):
        got_c, got_p = c.step(4, step), p.step(4, step)
        same_selection(got_p, got_c, f"step {step}")
    got_p0 = p.step(4, 0)
    compare(got_p0, oracle_step(x, N, 4, 0), x, dtype, check_tau=True)


DENSE = [
    # B, h_q, h_k, h_v, d_k, d_v, lens, dtype
    (1, 12, 2, 2, 64, 128, [5000], "bf16"),
    (2, 32, 4, 8, 32, 64, [3000, 17], "bf16"),
    (3, 4, 1, 1, 32, 64, [1, 0, 700], "f32"),
    (1, 12, 2, 4, 64, 128, [2049], "bf16"),
]


@pytest.mark.parametrize("case", range(len(DENSE)))
def test_reduced_key_dim_dense(case):
    B, h_q, h_k, h_v, dk, dv, lens, dtype = DENSE[case]
    say(f"dense case {case}: {DENSE[case]}")
    x = small(B, h_q, h_k, h_v, dk, dv, lens, dtype, seed=40 + case)
    l_kv = torch.from_numpy(x.l_kv).to(DEV)
    out = api.dense_gqa_attn(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), l_kv, out_dtype=torch.float32)
    pk = wl.paginate(x.k, x.v, x.l_kv, 32, seed=case, stale=-3)
    paged = api.dense_gqa_attn_paged(x.q.to(DEV), pk.k_pages.to(DEV), pk.v_pages.to(DEV), pk.table.to(DEV), l_kv,
                                     max_l_kv=x.k.shape[2], out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert got.shape == (B, h_q, dv)
    assert np.array_equal(paged.double().cpu().numpy(), got)
    q64, k64, v64 = x.f64()
    ref = orc.dense_gqa(q64, k64, v64, x.l_kv)
    tol = 1e-5 if dtype == "f32" else 2e-3
    for b in range(B):
        if x.l_kv[b] == 0:
            assert np.all(got[b] == 0)
            continue
        for j in range(h_q):
            assert np.abs(got[b, j] - ref[b, j]).max() <= tol * np.abs(ref[b, j]).max(), (b, j)
