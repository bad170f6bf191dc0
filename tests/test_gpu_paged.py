"""Paged (non-contiguous) caches: the paged entry points against the contiguous ones
and against the CPU oracle, on identical seeded inputs (needs an MI355X).

The paged layout only changes where token rows live: with the same chunks the
logits, thresholds, kept sets (in their fixed slot order), counts and outputs must
equal the contiguous call's bit for bit.
Page ids of pages past a sequence's length are set to out-of-range values, which
the library must never use for results.
"""
import numpy as np
import pytest
import torch

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import DERIVED, GpuCase, compare, out_bound

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[paged] {msg}", flush=True)


def small(B, h_q, h_k, h_v, d, lens, dtype, seed, l_max=None, plant=0.01):
    w = wl.Workload("small-paged", 190 + seed, batch=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, l_kv=max(lens), N=1,
                    refresh_period=1, dtype=dtype, plant_frac=plant)
    return wl.generate(w, seed=seed, lengths=lens, l_max=l_max or max(max(lens), 1))


class PagedCase:
    """Device copies of paged caches plus the outputs of one paged decode call."""

    def __init__(self, x, N, page_tokens, stale, seed, sel_cap, max_l_kv):
        pk = wl.paginate(x.k, x.v, x.l_kv, page_tokens, seed=seed, stale=stale)
        self.kp, self.vp, self.table = pk.k_pages.to(DEV), pk.v_pages.to(DEV), pk.table.to(DEV)
        self.q = x.q.to(DEV)
        self.l_kv = torch.from_numpy(np.asarray(x.l_kv, np.int32)).to(DEV)
        B, h_q, _ = x.q.shape
        self.N, self.max_l_kv, self.cap = N, max_l_kv, sel_cap
        self.tau = torch.zeros(B, h_q, dtype=torch.float32, device=DEV)
        self.out = torch.empty(B, h_q, x.v.shape[3], dtype=torch.float32, device=DEV)
        self.sel_count = torch.zeros(B, h_q, dtype=torch.int32, device=DEV)
        self.sel_idx = torch.full((B, h_q, sel_cap), -1, dtype=torch.int32, device=DEV)
        self.flags = torch.full((B, h_q), -1, dtype=torch.int32, device=DEV)

    def step(self, refresh_period, step, tau_in=None):
        if tau_in is not None:
            self.tau.copy_(torch.as_tensor(np.asarray(tau_in, np.float32)))
        self.sel_idx.fill_(-1)
        api.decode_attn_paged(self.q, self.kp, self.vp, self.table, self.l_kv, self.tau, N=self.N,
                              refresh_period=refresh_period, step=step, max_l_kv=self.max_l_kv, out=self.out,
                              sel_count=self.sel_count, sel_idx=self.sel_idx, flags=self.flags)
        torch.cuda.synchronize()
        return dict(O=self.out.double().cpu().numpy(), tau=self.tau.double().cpu().numpy(),
                    count=self.sel_count.cpu().numpy(), idx=self.sel_idx.cpu().numpy(),
                    flags=self.flags.cpu().numpy())


def same_selection(p, c, where, same_form=True):
    """Paged result p equals contiguous result c: bit for bit when both take the same
    value-gather form; otherwise (the contiguous call gathers late, the paged call
    early) the thresholds, counts, flags and kept sets bit for bit, and the outputs,
    summed in another order, within the derived bound of the arithmetic."""
    assert np.array_equal(p["tau"], c["tau"]), f"{where}: thresholds differ"
    assert np.array_equal(p["count"], c["count"]), f"{where}: counts differ"
    assert np.array_equal(p["flags"], c["flags"]), f"{where}: flags differ"
    if same_form:
        assert np.array_equal(p["idx"], c["idx"]), f"{where}: kept indices differ"
        assert np.array_equal(p["O"], c["O"]), f"{where}: outputs differ"
        return
    cap = p["idx"].shape[-1]
    for r in np.ndindex(p["count"].shape):
        n = min(int(p["count"][r]), cap)
        assert np.array_equal(np.sort(p["idx"][r][:n]), np.sort(c["idx"][r][:n])), f"{where}: kept sets differ at {r}"
    err = np.abs(p["O"] - c["O"]).max(axis=-1) / np.maximum(np.abs(c["O"]).max(axis=-1), 1e-30)
    assert err.max() <= DERIVED, f"{where}: outputs differ by {err.max():.2e}"


PAGED = [
    # B, h_q, h_k, h_v, d, lens, l_max, dtype, N, page_tokens, stale page id
    (2, 8, 2, 4, 64, [1000, 37], None, "bf16", 16, 16, -1),
    (3, 12, 1, 4, 128, [513, 1, 2000], None, "bf16", 32, 64, 10 ** 9),
    (1, 12, 1, 4, 128, [3000], 4096, "bf16", 32, 256, -1),     # one sequence: speculative key loads
    (1, 32, 2, 8, 64, [4097], None, "bf16", 64, 1024, -7),
    (2, 4, 1, 4, 64, [300, 65], None, "f32", 8, 32, -1),
    (1, 16, 1, 16, 128, [777], 1024, "f32", 20, 128, 2 ** 31 - 1),
    (2, 8, 4, 2, 128, [3000, 2999], None, "bf16", 7, 512, -1),
    (2, 6, 6, 6, 64, [100, 64], None, "bf16", 100, 16, -1),
]


@pytest.mark.parametrize("case", range(len(PAGED)))
def test_paged_equals_contiguous_and_oracle(case):
    B, h_q, h_k, h_v, d, lens, l_max, dtype, N, pt, stale = PAGED[case]
    say(f"case {case}: {PAGED[case]}")
    x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=case, l_max=l_max)
    max_l_kv = x.k.shape[2]
    cap = min(max_l_kv, max(4 * N, 64))
    c = GpuCase(x, N, sel_cap=cap)
    p = PagedCase(x, N, pt, stale, seed=case, sel_cap=cap, max_l_kv=max_l_kv)
    # refresh step, then a step that reuses each side's threshold
    got_c, got_p = c.step(4, 0), p.step(4, 0)
    same_selection(got_p, got_c, "refresh step")
    q64, k64, v64 = x.f64()
    ref = orc.saga_decode_step(q64, k64, v64, x.l_kv, N, 4, 0)
    compare(got_p, ref, x, dtype, check_tau=True)
    got_c1, got_p1 = c.step(4, 1), p.step(4, 1)
    same_selection(got_p1, got_c1, "stale step")
    # a stale threshold that keeps nothing: the forced exact refresh reads the pages too
    tau_inf = np.full((B, h_q), np.inf, np.float32)
    got_c2, got_p2 = c.step(4, 2, tau_in=tau_inf), p.step(4, 2, tau_in=tau_inf)
    same_selection(got_p2, got_c2, "forced refresh")
    live = np.asarray(lens) > 0
    assert np.all(got_p2["flags"][live] == 3)


def test_paged_batch16_full_size():
    # the batch-16, 128K Qwen-shaped workload in 256-token pages (one page per chunk)
    w = wl.QWEN_128K_B16
    x = wl.generate(w, seed=0)
    say(f"{w.name}: paged, 256-token pages")
    c = GpuCase(x, w.N, sel_cap=4 * w.N)
    p = PagedCase(x, w.N, 256, -1, seed=1, sel_cap=4 * w.N, max_l_kv=x.k.shape[2])
    # paged calls always gather early; the contiguous call takes the form of its shape
    same = api.gather_form(api.make_shape(c.q, c.k, c.v), w.N, x.k.shape[2]) == "early"
    for step in (0, 1):
        same_selection(p.step(w.refresh_period, step), c.step(w.refresh_period, step), f"step {step}", same)


DENSE_PAGED = [
    # B, h_q, h_k, h_v, d, lens, dtype, page_tokens
    (1, 12, 2, 2, 128, [5000], "bf16", 256),
    (2, 32, 8, 8, 64, [3000, 17], "bf16", 16),
    (3, 4, 1, 1, 64, [1, 0, 700], "f32", 64),
    (1, 12, 1, 4, 128, [5000], "bf16", 1024),
    (2, 32, 2, 8, 64, [3000, 1], "bf16", 32),
]


@pytest.mark.parametrize("case", range(len(DENSE_PAGED)))
def test_dense_paged(case):
    B, h_q, h_k, h_v, d, lens, dtype, pt = DENSE_PAGED[case]
    say(f"dense case {case}: {DENSE_PAGED[case]}")
    x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=60 + case)
    l_kv = torch.from_numpy(x.l_kv).to(DEV)
    pk = wl.paginate(x.k, x.v, x.l_kv, pt, seed=case, stale=-3)
    got = api.dense_gqa_attn_paged(x.q.to(DEV), pk.k_pages.to(DEV), pk.v_pages.to(DEV), pk.table.to(DEV), l_kv,
                                   max_l_kv=x.k.shape[2], out_dtype=torch.float32)
    cont = api.dense_gqa_attn(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), l_kv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got, cont = got.double().cpu().numpy(), cont.double().cpu().numpy()
    # the dense kernels sum in a fixed order: the paged call is bit-identical
    assert np.array_equal(got, cont)
    q64, k64, v64 = x.f64()
    ref = orc.dense_gqa(q64, k64, v64, x.l_kv)
    tol = out_bound(dtype)
    for b in range(B):
        if x.l_kv[b] == 0:
            assert np.all(got[b] == 0)
            continue
        for j in range(h_q):
            assert np.abs(got[b, j] - ref[b, j]).max() <= tol * np.abs(ref[b, j]).max(), (b, j)
