"""Contexts of 2^20 and 2^21 + 1000 keys, eight and sixteen times the pages' longest
(needs an MI355X).

The Qwen2.5-1.5B-shaped layer (h_q=12, h_k=1, h_v=4, d=128, bf16, N=512) at
l_kv = 1,048,576: 2048 chunks of 512 keys (8 tiles per wave) in one sequence, with
speculative key loads and a combine over 2048 chunk records per row. The oracle is evaluated row by row (every one of the 12
rows) for the decode step and for the dense kernels (SAGA with full attention
over all 2^20 keys). The 2^21 + 1000 case has more than 4096 chunks per row, where
the refresh collects its threshold candidates per slice of 4096 logits.
"""
import numpy as np
import pytest
import torch

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import DERIVED, GpuCase, check_sampled_rows

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
W_1M = wl.QWEN_128K.with_(name="qwen2.5-1.5b-shape-l1m", workload_id=9, l_kv=1 << 20)


def say(msg):
    print(f"[long context] {msg}", flush=True)


@pytest.fixture(scope="module")
def inputs():
    say(f"generating {W_1M.name}")
    return wl.generate(W_1M, seed=0)


def test_decode_step_1m_keys(inputs):
    x, w = inputs, W_1M
    g = GpuCase(x, w.N)
    say("refresh step, then two steps reusing the threshold")
    got0 = g.step(w.refresh_period, 0)
    got1 = g.step(w.refresh_period, 1)
    got2 = g.step(w.refresh_period, 7)
    assert np.all(got0["flags"] == 1) and np.all(got1["flags"] == 0)
    assert np.array_equal(got1["count"], got0["count"]) and np.array_equal(got2["count"], got0["count"])
    check_sampled_rows(x, w.N, [(0, j) for j in range(w.h_q)], [got0, got1, got2], w.dtype)


def test_dense_1m_keys(inputs):
    x, w = inputs, W_1M
    say("dense SAGA attention over every key")
    l_kv = torch.from_numpy(x.l_kv).to(DEV)
    out = api.dense_gqa_attn(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), l_kv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    scale = 1.0 / np.sqrt(w.d)
    L = int(x.l_kv[0])
    K = x.k[0, 0, :L].double().numpy()
    for vg in range(w.h_v):
        V = x.v[0, vg, :L].double().numpy()
        for j in range(w.h_q):
            if orc.value_head_of(j, w.h_q, w.h_v) != vg:
                continue
            a = orc.attention_logits(x.q[0, j].double().numpy(), K, scale)
            ref, _ = orc.sparse_softmax_pv(a, V)
            assert np.abs(got[0, j] - ref).max() <= DERIVED * np.abs(ref).max(), j
        del V


# Past 4096 chunks per row (2^21 + 1000 keys in chunks of 512) the refresh collects its
# threshold candidates in slices of 4096 logits (k_cand_collect) instead of per chunk.
W_2M = wl.QWEN_128K.with_(name="qwen2.5-1.5b-shape-l2m", workload_id=10, l_kv=(1 << 21) + 1000)


def test_decode_step_slice_candidates_2m_keys():
    w = W_2M
    say(f"generating {w.name}")
    x = wl.generate(w, seed=0)
    g = GpuCase(x, w.N)
    say("refresh step (candidates per slice), then a step reusing the threshold")
    got0 = g.step(w.refresh_period, 0)
    got1 = g.step(w.refresh_period, 1)
    assert np.all(got0["flags"] == 1) and np.all(got1["flags"] == 0)
    assert np.array_equal(got1["count"], got0["count"])
    check_sampled_rows(x, w.N, [(0, 0), (0, 5), (0, 11)], [got0, got1], w.dtype)
