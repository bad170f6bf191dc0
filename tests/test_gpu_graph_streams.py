"""The decode step under HIP graph capture and on concurrent streams (needs an MI355X).

The library enqueues only kernels on the caller's stream (no allocation, copy, fill
or synchronisation), and every call leaves the workspace counters it uses at zero,
so a captured sequence of decode steps can be replayed. These tests replay a
captured sequence several times, with eager work in between, and check every replay
against the same steps run eagerly (whose last step is checked against the oracle);
and they run two decode sequences with separate workspaces on two streams at once,
each checked against the same sequence run alone.

Kept entries take fixed slots and every sum runs in a fixed order, so a replay or a
concurrent run gives the same bits as the eager run: thresholds, counts, flags, the
exported kept indices (in their order) and the outputs are compared exactly.
"""
import numpy as np
import pytest
import torch

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import compare

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[graph/streams] {msg}", flush=True)


def inputs(seed, B, h_q, h_k, h_v, d, lens, dtype="bf16"):
    w = wl.Workload("graph-streams", 490 + seed, batch=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, l_kv=max(lens), N=1,
                    refresh_period=1, dtype=dtype, plant_frac=0.01)
    return wl.generate(w, seed=seed, lengths=lens, l_max=max(lens))


class Steps:
    """Device buffers for a sequence of decode steps; each step writes its own outputs."""

    def __init__(self, x, N, period, steps):
        self.x, self.N, self.period, self.steps = x, N, period, steps
        self.q, self.k, self.v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
        self.l_kv = torch.from_numpy(np.asarray(x.l_kv, np.int32)).to(DEV)
        B, h_q, _ = x.q.shape
        self.L = int(x.k.shape[2])
        self.cap = min(self.L, 4 * N)
        self.tau = torch.zeros(B, h_q, dtype=torch.float32, device=DEV)
        self.out = torch.zeros(steps, B, h_q, x.v.shape[3], dtype=torch.float32, device=DEV)
        self.tau_t = torch.zeros(steps, B, h_q, dtype=torch.float32, device=DEV)
        self.count = torch.zeros(steps, B, h_q, dtype=torch.int32, device=DEV)
        self.idx = torch.full((steps, B, h_q, self.cap), -1, dtype=torch.int32, device=DEV)
        self.flags = torch.zeros(steps, B, h_q, dtype=torch.int32, device=DEV)
        self.ws = api.Workspace(api.make_shape(self.q, self.k, self.v, torch.float32), N, self.L, DEV)

    def run(self, stream=None):
        """Enqueue every step on the current stream (or `stream`); no host synchronisation."""
        for t in range(self.steps):
            api.decode_attn(self.q, self.k, self.v, self.l_kv, self.tau, N=self.N, refresh_period=self.period,
                            step=t, max_l_kv=self.L, out=self.out[t], sel_count=self.count[t], sel_idx=self.idx[t],
                            flags=self.flags[t], workspace=self.ws, stream=stream)
            self.tau_t[t].copy_(self.tau)

    def clear(self):
        self.out.zero_()
        self.tau_t.zero_()
        self.count.zero_()
        self.idx.fill_(-1)
        self.flags.zero_()

    def result(self):
        return dict(O=self.out.double().cpu().numpy(), tau=self.tau_t.double().cpu().numpy(),
                    count=self.count.cpu().numpy(), idx=self.idx.cpu().numpy(), flags=self.flags.cpu().numpy())


def same_steps(got, ref, where):
    assert np.array_equal(got["tau"], ref["tau"]), f"{where}: thresholds differ"
    assert np.array_equal(got["count"], ref["count"]), f"{where}: counts differ"
    assert np.array_equal(got["flags"], ref["flags"]), f"{where}: flags differ"
    assert np.array_equal(got["idx"], ref["idx"]), f"{where}: kept indices differ"
    assert np.array_equal(got["O"], ref["O"]), f"{where}: outputs differ"


@pytest.mark.parametrize("case", [
    # B, h_q, h_k, h_v, d, lens, N, period, steps, value-gather form
    (2, 12, 1, 4, 128, [5000, 1777], 64, 4, 9, "early"),
    (3, 32, 2, 8, 64, [3000, 0, 4096], 32, 3, 7, "early"),
    (2, 12, 1, 4, 128, [65536, 40000], 128, 4, 5, "late"),   # 512 select blocks, < 1 kept per chunk
])
def test_graph_replays_equal_eager_steps(case):
    B, h_q, h_k, h_v, d, lens, N, period, steps, form = case
    say(f"graph case {case}")
    x = inputs(1, B, h_q, h_k, h_v, d, lens)
    st = Steps(x, N, period, steps)
    assert api.gather_form(api.make_shape(st.q, st.k, st.v), N, st.L) == form
    st.run()
    torch.cuda.synchronize()
    ref = st.result()
    # the eager steps follow the oracle: the last step against the oracle's multi-step rule
    q64, k64, v64 = x.f64()
    tau_o = None
    for t in range(steps):
        r = orc.saga_decode_step(q64, k64, v64, x.l_kv, N, period, t, tau_in=tau_o)
        tau_o = r.tau
    last = {k: ref[k][steps - 1] for k in ("O", "count", "idx", "flags")}
    last["tau"] = ref["tau"][steps - 1]
    compare(last, r, x, "bf16", check_tau=((steps - 1) % period == 0))

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    st.clear()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        st.run()
    torch.cuda.synchronize()
    other = inputs(2, B, h_q, h_k, h_v, d, lens)
    eager = Steps(other, N, period, 2)
    for rep in range(3):
        st.clear()
        st.tau.zero_()                                # the eager sequence's starting state
        g.replay()
        torch.cuda.synchronize()
        same_steps(st.result(), ref, f"replay {rep}")
        eager.run()                                   # eager work on the same device between replays
        torch.cuda.synchronize()


def test_two_streams_two_workspaces():
    a = Steps(inputs(3, 2, 12, 1, 4, 128, [6000, 2500]), 64, 4, 6)
    b = Steps(inputs(4, 1, 32, 2, 8, 64, [7000]), 32, 2, 6)
    a.run()
    b.run()
    torch.cuda.synchronize()
    ref_a, ref_b = a.result(), b.result()
    a.clear()
    b.clear()
    a.tau.zero_()
    b.tau.zero_()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    say("two decode sequences on two streams")
    for t in range(a.steps):                          # interleaved enqueue, one sequence per stream
        with torch.cuda.stream(sa):
            api.decode_attn(a.q, a.k, a.v, a.l_kv, a.tau, N=a.N, refresh_period=a.period, step=t, max_l_kv=a.L,
                            out=a.out[t], sel_count=a.count[t], sel_idx=a.idx[t], flags=a.flags[t], workspace=a.ws)
            a.tau_t[t].copy_(a.tau)
        with torch.cuda.stream(sb):
            api.decode_attn(b.q, b.k, b.v, b.l_kv, b.tau, N=b.N, refresh_period=b.period, step=t, max_l_kv=b.L,
                            out=b.out[t], sel_count=b.count[t], sel_idx=b.idx[t], flags=b.flags[t], workspace=b.ws)
            b.tau_t[t].copy_(b.tau)
    torch.cuda.synchronize()
    same_steps(a.result(), ref_a, "stream a")
    same_steps(b.result(), ref_b, "stream b")
