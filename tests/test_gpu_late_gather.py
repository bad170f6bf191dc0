"""GPU parity of the late value gather (slot records read by the combining kernel)
away from its usual one kept entry per chunk.

The shape takes the late form: two Qwen-shaped sequences of 65536 keys (h_q=12,
h_k=1, h_v=4, d=128, bf16, N=256): 256-key chunks, 512 select blocks. Stale
thresholds then keep from a few to every key of a row, so records overflow their
seven inline entries into the chunk's segment of the kept list; a row whose
threshold keeps nothing takes the forced refresh through the combining kernel.
Every result is compared with the oracle (tests/parity.py rules), and repeated
steps must give the same bits. Further shapes that take the late form cover the
kernel's other instantiations: fp32 caches with 64- and 128-wide heads (16 and 32
blocks per row), and 64-wide keys with 128-wide values.
"""
import numpy as np
import pytest
import torch

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import GpuCase, compare

pytestmark = pytest.mark.gpu

L, N = 65536, 256


def say(msg):
    print(f"[late-gather] {msg}", flush=True)


def inputs(seed):
    w = wl.Workload("late-gather", 300 + seed, batch=2, h_q=12, h_k=1, h_v=4, d=128, l_kv=L, N=N,
                    refresh_period=1, dtype="bf16", plant_frac=0.005)
    return wl.generate(w, seed=seed, lengths=[L, L])


def row_quantiles(x, keep):
    """Per (b, j) the float32 logit below which a fraction 1 - keep of the row lies."""
    q64, k64, _ = x.f64()
    B, h_q, d = q64.shape
    h_k = k64.shape[1]
    tau = np.empty((B, h_q), np.float32)
    for b in range(B):
        for j in range(h_q):
            a = orc.attention_logits(q64[b, j], k64[b, orc.key_head_of(j, h_q, h_k), :L], 1.0 / np.sqrt(d))
            tau[b, j] = np.float32(np.quantile(a, 1.0 - keep))
    return tau


def test_shape_takes_the_late_form():
    x = inputs(0)
    g = GpuCase(x, N)
    assert api.gather_form(api.make_shape(g.q, g.k, g.v), N, L) == "late"


@pytest.mark.parametrize("keep", [0.002, 0.03, 0.25])
def test_stale_thresholds_keeping_many_entries_per_chunk(keep):
    say(f"stale thresholds keeping {keep:.1%} of each row")
    x = inputs(1)
    g = GpuCase(x, N, sel_cap=L)
    tau_in = row_quantiles(x, keep)
    tau_in[0, 3] = np.inf     # keeps nothing: forced exact refresh
    tau_in[1, 7] = -np.inf    # keeps every key: 256 entries per record
    runs = [g.step(1 << 20, 5, tau_in=tau_in) for _ in range(2)]
    for key in ("O", "tau", "count", "idx", "flags"):
        assert np.array_equal(runs[0][key], runs[1][key]), key
    q64, k64, v64 = x.f64()
    ref = orc.saga_decode_step(q64, k64, v64, x.l_kv, N, 1 << 20, 5, tau_in=tau_in.astype(np.float64))
    compare(runs[0], ref, x, "bf16", check_tau=True)
    assert runs[0]["flags"][0, 3] == 3 and runs[0]["count"][0, 3] == N
    assert runs[0]["count"][1, 7] == L
    # the kept indices are exported in key order
    for b in range(2):
        for j in range(12):
            n = int(runs[0]["count"][b, j])
            assert np.all(np.diff(runs[0]["idx"][b, j, :n]) > 0), (b, j)


def test_refresh_step_then_stale_steps():
    say("refresh step, then steps reusing its thresholds")
    x = inputs(2)
    g = GpuCase(x, N, sel_cap=4 * N)
    q64, k64, v64 = x.f64()
    r0 = g.step(4, 0)
    ref0 = orc.saga_decode_step(q64, k64, v64, x.l_kv, N, 4, 0)
    compare(r0, ref0, x, "bf16", check_tau=True)
    r1 = g.step(4, 1)
    ref1 = orc.saga_decode_step(q64, k64, v64, x.l_kv, N, 4, 1, tau_in=ref0.tau)
    compare(r1, ref1, x, "bf16", check_tau=False)
    assert np.array_equal(r1["count"], r0["count"])
    torch.cuda.synchronize()


LATE_SHAPES = [
    # B, h_q, h_k, h_v, d, d_v, L, N, dtype
    (1, 4, 1, 4, 64, 64, 131072, 256, "f32"),     # 256-byte fp32 value rows
    (1, 4, 1, 2, 128, 128, 131072, 256, "f32"),   # 512-byte fp32 value rows
    (4, 12, 1, 4, 64, 128, 65536, 128, "bf16"),   # 64-wide keys, 128-wide values, 512-key chunks
]


@pytest.mark.parametrize("case", range(len(LATE_SHAPES)))
def test_other_late_instantiations(case):
    B, h_q, h_k, h_v, d, dv, Lc, Nc, dtype = LATE_SHAPES[case]
    say(f"late form at {LATE_SHAPES[case]}")
    w = wl.Workload("late-gather-shapes", 310 + case, batch=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, d_v=dv, l_kv=Lc, N=Nc,
                    refresh_period=1, dtype=dtype, plant_frac=0.005)
    x = wl.generate(w, seed=case, lengths=[Lc] * B)
    g = GpuCase(x, Nc, sel_cap=4 * Nc)
    assert api.gather_form(api.make_shape(g.q, g.k, g.v), Nc, Lc) == "late"
    q64, k64, v64 = x.f64()
    r0 = g.step(4, 0)
    ref0 = orc.saga_decode_step(q64, k64, v64, x.l_kv, Nc, 4, 0)
    compare(r0, ref0, x, dtype, check_tau=True)
    r1 = g.step(4, 1)
    ref1 = orc.saga_decode_step(q64, k64, v64, x.l_kv, Nc, 4, 1, tau_in=ref0.tau)
    compare(r1, ref1, x, dtype, check_tau=False)


def test_stage_entry_points_equal_the_step_in_the_late_form():
    say("saga_select_gather + saga_split_combine against the step, late form")
    x = inputs(3)
    g = GpuCase(x, N, sel_cap=4 * N)
    g.step(4, 0)
    ref = g.step(4, 1)                      # a step reusing the threshold of step 0
    tau = g.tau.clone()
    out = torch.empty_like(g.out)
    cnt = torch.zeros_like(g.sel_count)
    idx = torch.full_like(g.sel_idx, -1)
    api.select_gather(g.q, g.k, g.v, g.l_kv, tau, N=N, max_l_kv=g.max_l_kv, workspace=g.ws)
    api.split_combine(g.q, g.k, g.v, g.l_kv, tau, N=N, max_l_kv=g.max_l_kv, out=out, sel_count=cnt, sel_idx=idx,
                      workspace=g.ws)
    torch.cuda.synchronize()
    # the same two launches as the step: the same bits
    assert np.array_equal(out.double().cpu().numpy(), ref["O"])
    assert np.array_equal(cnt.cpu().numpy(), ref["count"])
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
