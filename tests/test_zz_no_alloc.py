"""saga_decode_attn_noalloc (the decode step with the library's own per-GPU scratch)
against saga_decode_attn (the same step with a caller's workspace), through the
C ABI on the same inputs.

Three inputs in a row on one GPU, each smaller than the one before, each with a
refresh step and a step that reuses the threshold, so every later call runs on
scratch that still holds an earlier call's contents. The first (a Qwen-shaped
sequence of 128K) takes the late value gather, the other two the early one.
Thresholds, kept counts, flags, kept indices and outputs must be identical bit for
bit: the same kernels run on the same inputs, kept entries take fixed places and
every sum runs in a fixed order. The first two inputs are also checked against the
CPU oracle with the bar of the parity tests.
"""
import numpy as np
import pytest
import torch

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl

DEV = torch.device("cuda:0")
pytestmark = pytest.mark.gpu

FIRST = wl.QWEN_128K.with_(refresh_period=4)
MIDDLE = wl.QWEN_128K.with_(l_kv=32768, N=256, refresh_period=4)
SECOND = wl.LLAMA_32K.with_(h_q=8, h_k=2, h_v=4, l_kv=3000, N=64, refresh_period=3)


class Side:
    """Threshold state and outputs of one entry point."""

    def __init__(self, B, h_q, d_v, cap):
        self.tau = torch.zeros(B, h_q, dtype=torch.float32, device=DEV)
        self.out = torch.full((B, h_q, d_v), 123.0, dtype=torch.float32, device=DEV)
        self.count = torch.full((B, h_q), -1, dtype=torch.int32, device=DEV)
        self.idx = torch.full((B, h_q, cap), -1, dtype=torch.int32, device=DEV)
        self.flags = torch.full((B, h_q), -1, dtype=torch.int32, device=DEV)


def run_pair(w, steps):
    x = wl.generate(w, seed=3)
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    l_kv = torch.from_numpy(x.l_kv).to(DEV)
    B, h_q, _ = x.q.shape
    cap = 4 * w.N
    ref, na = Side(B, h_q, w.dv, cap), Side(B, h_q, w.dv, cap)
    ws = api.Workspace(api.make_shape(q, k, v, torch.float32), w.N, int(k.shape[2]), DEV)
    results = []
    for t in steps:
        api.decode_attn(q, k, v, l_kv, ref.tau, N=w.N, refresh_period=w.refresh_period, step=t, out=ref.out,
                        sel_count=ref.count, sel_idx=ref.idx, flags=ref.flags, workspace=ws)
        api.decode_attn_noalloc(q, k, v, l_kv, na.tau, N=w.N, refresh_period=w.refresh_period, step=t, out=na.out,
                                sel_count=na.count, sel_idx=na.idx, flags=na.flags)
        torch.cuda.synchronize()
        assert torch.equal(ref.tau, na.tau), t
        assert torch.equal(ref.count, na.count), t
        assert torch.equal(ref.flags, na.flags), t
        assert int(ref.count.max()) <= cap
        assert torch.equal(ref.idx, na.idx), t
        assert torch.equal(ref.out, na.out), t
        results.append((x, t, na.out.double().cpu().numpy(), na.tau.double().cpu().numpy(),
                        na.count.cpu().numpy(), na.flags.cpu().numpy()))
    return results


def form(w):
    shape = api.SagaShape(w.batch, w.h_q, w.h_k, w.h_v, w.d, 0, w.l_kv, api.BF16, api.F32, 0.0)
    return api.gather_form(shape, w.N, w.l_kv)


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    assert (form(FIRST), form(MIDDLE), form(SECOND)) == ("late", "early", "early")
    first = run_pair(FIRST, steps=[0, 1])
    middle = run_pair(MIDDLE, steps=[0, 1])
    second = run_pair(SECOND, steps=[0, 2])
    assert SECOND.l_kv * SECOND.h_q < MIDDLE.l_kv * MIDDLE.h_q < FIRST.l_kv * FIRST.h_q
    # the refresh steps of the first two inputs against the oracle (exact top-N at a refresh)
    for res, w in ((first, FIRST), (middle, MIDDLE)):
        x, t, out, tau, count, flags = res[0]
        q64, k64, v64 = x.f64()
        r = orc.saga_decode_step(q64, k64, v64, x.l_kv, w.N, w.refresh_period, t)
        s = np.maximum(np.abs(r.tau), 1.0)
        assert np.all(np.abs(tau - r.tau) <= 1e-5 * s)
        err = (np.abs(out - r.O).max(axis=-1) / np.abs(r.O).max(axis=-1)).max()
        assert err <= 1e-5, err  # exact bf16 inputs, fp32 arithmetic and outputs
        assert np.all(flags == 1)
    # every input: every row kept at least N entries at its refresh step
    for res, w in ((first, FIRST), (middle, MIDDLE), (second, SECOND)):
        assert np.all(res[0][4] >= w.N)


def test_noalloc_refuses_a_step_larger_than_its_scratch():
    # four sequences of 128K need more than the scratch holds: refused before any launch
    B, h_q, h_k, h_v, d, L = 4, 12, 1, 4, 128, 131072
    shape = api.SagaShape(B, h_q, h_k, h_v, d, 0, L, api.BF16, api.F32, 0.0)
    assert api.workspace_bytes(shape, 512, L) > api.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, h_q, d, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, h_k, L, d, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(B, h_v, L, d, dtype=torch.bfloat16, device=DEV)
    l_kv = torch.full((B,), L, dtype=torch.int32, device=DEV)
    tau = torch.full((B, h_q), 7.0, dtype=torch.float32, device=DEV)
    out = torch.full((B, h_q, d), 5.0, dtype=torch.float32, device=DEV)
    with pytest.raises(api.SagaError) as e:
        api.decode_attn_noalloc(q, k, v, l_kv, tau, N=512, refresh_period=32, step=0, out=out)
    assert e.value.status == api.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 5.0) and torch.all(tau == 7.0)
