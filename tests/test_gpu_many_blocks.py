"""Launches with many chunk blocks against the CPU oracle (needs an MI355X).

Each case gives the select kernel at least 2048 chunk blocks (chunks x key heads x
head splits x sequences; the comments give the count) at a size the oracle finishes
in seconds: many key heads, heads split over many blocks per chunk, fp32 chunks
of 512 keys. The lengths are ragged so that some blocks hold no keys (an empty sequence,
a sequence of one key) and the last chunk of a sequence is partly past its length.
Stale, forced and mixed thresholds are checked, and paged caches against the
contiguous ones.
"""
import numpy as np
import pytest

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import GpuCase, compare
from tests.test_gpu_paged import PagedCase, same_selection

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[many blocks] {msg}", flush=True)


def small(B, h_q, h_k, h_v, d, lens, dtype, seed, l_max):
    w = wl.Workload("small-many-blocks", 390 + seed, batch=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, l_kv=max(lens), N=1,
                    refresh_period=1, dtype=dtype, plant_frac=0.01)
    return wl.generate(w, seed=seed, lengths=lens, l_max=l_max)


def oracle_step(x, N, n, step, tau_in=None):
    q64, k64, v64 = x.f64()
    return orc.saga_decode_step(q64, k64, v64, x.l_kv, N, n, step, tau_in=tau_in)


CASES = [
    # B, h_q, h_k, h_v, d, lens, l_max, dtype, N
    # 64 chunks of 256 keys x 12 blocks per chunk (half the keys kept: the 12 heads of
    # the key head are split over 12 blocks) x 4 sequences = 3072 blocks
    (4, 12, 1, 4, 128, [16384, 9000, 1, 16000], 16384, "bf16", 8192),
    # 16 chunks of 512 keys x 32 key heads x 4 sequences = 2048 blocks
    (4, 64, 32, 32, 64, [8192, 0, 5000, 8191], 8192, "bf16", 64),
    # fp32 in chunks of 512 keys: 16 chunks x 64 key heads x 2 sequences = 2048 blocks
    (2, 64, 64, 64, 64, [8192, 3001], 8192, "f32", 32),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_many_chunk_blocks(case):
    B, h_q, h_k, h_v, d, lens, l_max, dtype, N = CASES[case]
    say(f"case {case}: {CASES[case]}")
    x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=case, l_max=l_max)
    g = GpuCase(x, N)
    got0 = g.step(4, 0)                      # refresh step: exact thresholds
    ref0 = oracle_step(x, N, 4, 0)
    compare(got0, ref0, x, dtype, check_tau=True)
    got1 = g.step(4, 1)                      # stale step: the threshold is reused
    compare(got1, oracle_step(x, N, 4, 1, tau_in=ref0.tau), x, dtype, check_tau=False)
    assert np.array_equal(got1["count"], got0["count"])
    # a stale threshold that keeps nothing: every live row takes the forced refresh
    tau_inf = np.full((B, h_q), np.inf, np.float32)
    got2 = g.step(4, 2, tau_in=tau_inf)
    compare(got2, oracle_step(x, N, 4, 2, tau_in=tau_inf.astype(np.float64)), x, dtype, check_tau=True)
    live = np.asarray(lens) > 0
    assert np.all(got2["flags"][live] == 3)
    # a threshold between the two: some rows keep entries, others are forced
    tau_mix = np.where(np.arange(h_q)[None, :] % 2 == 0, ref0.tau, np.inf).astype(np.float32)
    got3 = g.step(4, 3, tau_in=tau_mix)
    compare(got3, oracle_step(x, N, 4, 3, tau_in=tau_mix.astype(np.float64)), x, dtype, check_tau=True)


@pytest.mark.parametrize("page_tokens", [16, 512])
def test_many_chunk_blocks_paged(page_tokens):
    # case 1 in pages smaller than a chunk and as large as one: the same selection
    B, h_q, h_k, h_v, d, lens, l_max, dtype, N = CASES[1]
    say(f"paged, {page_tokens}-token pages")
    x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=1, l_max=l_max)
    cap = 4 * N
    c = GpuCase(x, N, sel_cap=cap)
    p = PagedCase(x, N, page_tokens, -1, seed=2, sel_cap=cap, max_l_kv=l_max)
    for step in (0, 1):
        same_selection(p.step(4, step), c.step(4, step), f"step {step}")
