"""HIP path vs the CPU oracle on identical seeded inputs (needs an MI355X).

Sizes: small cases span several chunks and a ragged tail; the named workloads run
at full size in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

from oracle import saga_oracle as orc
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import DERIVED, GpuCase, check_sampled_rows, compare, out_bound

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[parity] {msg}", flush=True)


def oracle_step(x, N, n, step, tau_in=None):
    q64, k64, v64 = x.f64()
    return orc.saga_decode_step(q64, k64, v64, x.l_kv, N, n, step, tau_in=tau_in)


def small(B, h_q, h_k, h_v, d, lens, dtype, seed, plant=0.01, l_max=None):
    w = wl.Workload("small", 90 + seed, batch=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, l_kv=max(lens), N=1,
                    refresh_period=1, dtype=dtype, plant_frac=plant)
    return w, wl.generate(w, seed=seed, lengths=lens, l_max=l_max or max(max(lens), 1))


# --- the tiny fp32 workload: refresh every step == exact top-N ------------------

def test_tiny_fp32_exact_topn():
    w = wl.TINY
    x = wl.generate(w, seed=0)
    say(f"{w.name} N={w.N}")
    g = GpuCase(x, w.N)
    got = g.step(w.refresh_period, 0)
    ref = oracle_step(x, w.N, w.refresh_period, 0)
    compare(got, ref, x, "f32", check_tau=True)
    assert np.all(got["count"] == w.N)          # fp32 logits, no ties: exactly N kept
    assert np.all(got["flags"] == 1)
    # next step (refresh again) gives the same answer
    got2 = g.step(w.refresh_period, 1)
    assert np.array_equal(np.sort(got2["idx"], axis=-1), np.sort(got["idx"], axis=-1))


# --- small shapes: several chunks, ragged tails, head groupings ----------------

SMALL = [
    # B, h_q, h_k, h_v, d, lens, dtype, N
    (2, 8, 2, 4, 64, [1000, 37], "bf16", 16),
    (3, 12, 1, 4, 128, [513, 1, 2000], "bf16", 32),
    (1, 32, 2, 8, 64, [4097], "bf16", 64),
    (2, 4, 1, 4, 64, [300, 65], "f32", 8),
    (1, 16, 1, 16, 128, [777], "f32", 20),
    (1, 40, 1, 8, 64, [1500], "bf16", 10),
    (2, 6, 6, 6, 64, [100, 64], "bf16", 100),
    (2, 8, 4, 2, 128, [3000, 2999], "bf16", 7),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_shapes_refresh_and_stale(case):
    B, h_q, h_k, h_v, d, lens, dtype, N = SMALL[case]
    say(f"small case {case}: {SMALL[case]}")
    w, x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=case)
    g = GpuCase(x, N)
    got = g.step(4, 0)                            # refresh step
    ref = oracle_step(x, N, 4, 0)
    compare(got, ref, x, dtype, check_tau=True)
    assert np.all(got["flags"][np.array(lens) > 0] == 1)
    # stale step on the same inputs with each side's own threshold: same selection
    got1 = g.step(4, 1)
    ref1 = oracle_step(x, N, 4, 1, tau_in=ref.tau)
    compare(got1, ref1, x, dtype, check_tau=False)
    assert np.all(got1["flags"][np.array(lens) > 0] == 0)
    assert np.array_equal(got1["count"], got["count"])


# The chunk width follows the launch: the widest chunks (8, 4 or 2 tiles of 16 keys
# per wave) that still give two blocks per compute unit. The small shapes above take
# 2 tiles; these reach the wider forms at sizes the oracle finishes quickly.
CHUNK_FORMS = [
    # B, h_q, h_k, h_v, d, lens, dtype, N                                  tiles per wave
    (16, 12, 1, 4, 128, [16384, 1, 9000, 16383, 256, 511, 12000, 16384, 700, 16000, 3, 8192, 8193, 15000, 4097,
                         16384], "bf16", 64),                                # 8
    (8, 32, 2, 8, 128, [16384, 16000, 9000, 16384, 2049, 16384, 12345, 16384], "bf16", 2048),  # 8
    (16, 16, 1, 2, 128, [16384] * 16, "f32", 32),                          # 4 (32 KiB per wave)
    (4, 32, 2, 8, 64, [16384, 9000, 16383, 1], "bf16", 256),               # 4
]


@pytest.mark.parametrize("case", range(len(CHUNK_FORMS)))
def test_chunk_widths_refresh_and_stale(case):
    B, h_q, h_k, h_v, d, lens, dtype, N = CHUNK_FORMS[case]
    say(f"chunk form {case}: B={B} h_q={h_q} h_k={h_k} h_v={h_v} d={d} N={N} {dtype}")
    w, x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=50 + case)
    g = GpuCase(x, N, sel_cap=min(max(lens), 4 * N))
    got = g.step(4, 0)
    ref = oracle_step(x, N, 4, 0)
    compare(got, ref, x, dtype, check_tau=True)
    got1 = g.step(4, 1)
    ref1 = oracle_step(x, N, 4, 1, tau_in=ref.tau)
    compare(got1, ref1, x, dtype, check_tau=False)
    assert np.array_equal(got1["count"], got["count"])


def test_bf16_output_rounding():
    w, x = small(1, 12, 1, 4, 128, [5000], "bf16", seed=20)
    g = GpuCase(x, 64, out_dtype=torch.bfloat16)
    got = g.step(1, 0)
    compare(got, oracle_step(x, 64, 1, 0), x, "bf16", check_tau=True, out_bf16=True)


# --- named workloads at full size ------------------------------------------------

@pytest.mark.parametrize("name", ["llama3.2-1b-shape-l32k", "qwen2.5-1.5b-shape-l128k"])
def test_workload_full_size(name):
    w = wl.WORKLOADS[name]
    x = wl.generate(w, seed=0)
    say(f"{name}: refresh step then stale steps")
    g = GpuCase(x, w.N)
    got = g.step(w.refresh_period, 0)
    ref = oracle_step(x, w.N, w.refresh_period, 0)
    bands = compare(got, ref, x, w.dtype, check_tau=True)
    assert bands <= max(1, w.h_q // 8)
    got1 = g.step(w.refresh_period, 5)
    ref1 = oracle_step(x, w.N, w.refresh_period, 5, tau_in=ref.tau)
    compare(got1, ref1, x, w.dtype, check_tau=False)


def test_ragged_batch_full_size():
    w = wl.RAGGED_B8
    x = wl.generate(w, seed=0)
    say(f"{w.name}: lengths {x.l_kv.tolist()}")
    g = GpuCase(x, w.N)
    got = g.step(w.refresh_period, 0)
    ref = oracle_step(x, w.N, w.refresh_period, 0)
    bands = compare(got, ref, x, w.dtype, check_tau=True)
    assert bands <= 8
    got1 = g.step(w.refresh_period, 3)
    compare(got1, oracle_step(x, w.N, w.refresh_period, 3, tau_in=ref.tau), x, w.dtype, check_tau=False)


def test_batch16_full_size_sampled_rows():
    # 16 sequences of 128K: the oracle is evaluated row by row on a sample of
    # (sequence, head) rows spread over the batch (every row's threshold is its own)
    w = wl.QWEN_128K_B16
    x = wl.generate(w, seed=0)
    say(f"{w.name}: refresh step, then a stale step, sampled rows")
    g = GpuCase(x, w.N)
    got0 = g.step(w.refresh_period, 0)
    got1 = g.step(w.refresh_period, 1)
    rows = [(0, 0), (1, 11), (3, 5), (6, 8), (8, 2), (10, 9), (13, 4), (15, 7)]
    check_sampled_rows(x, w.N, rows, [got0, got1], w.dtype)
    assert np.array_equal(got0["count"], got1["count"])


# --- multi-step decode: appended rows, drifting query, periodic refresh ----------

def test_multistep_append_and_drift():
    w = wl.SWEEP.with_(N=128, refresh_period=8)
    s = wl.DecodeStream(w, seed=0, l0=4096, l_max=4096 + 40)
    g = GpuCase(s.inputs(), w.N, max_l_kv=4096 + 40)
    tau_o = None
    for t in range(24):
        x = s.inputs()
        g.refresh_inputs(x)
        got = g.step(w.refresh_period, t)
        ref = oracle_step(x, w.N, w.refresh_period, t, tau_in=tau_o)
        compare(got, ref, x, w.dtype, check_tau=(t % w.refresh_period == 0))
        assert np.all((got["flags"] & 1) == (1 if t % w.refresh_period == 0 else 0)) or ref.fallback.any()
        tau_o = ref.tau
        s.append(1)
        s.drift()


# --- the multi-step sweep grid: every context length, top-N size and period ------

SWEEP_GRID = [(L, N, n) for L in wl.SWEEP_L for N in wl.SWEEP_N for n in wl.SWEEP_PERIOD]


@pytest.mark.parametrize("L,N,n", SWEEP_GRID)
def test_sweep_grid_point(L, N, n):
    # four decode steps ending at context L (rows appended and q drifting between
    # steps), each side keeping its own threshold state
    say(f"sweep point l_kv={L} N={N} n={n}")
    w = wl.SWEEP.with_(N=N, refresh_period=n)
    s = wl.DecodeStream(w, seed=1, l0=L - 3, l_max=L)
    g = GpuCase(s.inputs(), N, max_l_kv=L)
    tau_o = None
    for t in range(4):
        x = s.inputs()
        if t:
            g.refresh_inputs(x)
        got = g.step(n, t)
        ref = oracle_step(x, N, n, t, tau_in=tau_o)
        compare(got, ref, x, w.dtype, check_tau=(t % n == 0))
        tau_o = ref.tau
        if t < 3:
            s.append(1)
            s.drift()


# --- forced paths ------------------------------------------------------------------

def test_empty_stale_selection_forces_refresh():
    w, x = small(2, 8, 2, 4, 128, [2500, 700], "bf16", seed=30)
    N = 24
    g = GpuCase(x, N, sel_cap=700)
    tau_in = np.full((2, 8), np.inf, np.float32)
    tau_in[1, 5] = -np.inf                        # this row keeps everything instead
    got = g.step(10, 3, tau_in=tau_in)
    ref = oracle_step(x, N, 10, 3, tau_in=tau_in.astype(np.float64))
    compare(got, ref, x, "bf16", check_tau=True)
    forced = ref.fallback
    assert forced.sum() == 15 and not forced[1, 5]
    assert np.all((got["flags"] == 3) == forced)
    assert got["count"][1, 5] == 700


def test_minus_inf_threshold_equals_dense():
    w, x = small(1, 4, 1, 4, 64, [900], "f32", seed=31)
    g = GpuCase(x, 8, sel_cap=900)
    got = g.step(5, 2, tau_in=np.full((1, 4), -np.inf, np.float32))
    q64, k64, v64 = x.f64()
    dense = orc.saga_decode_step(q64, k64, v64, x.l_kv, N=10 ** 6, refresh_period=1, step=0)
    assert np.all(got["count"] == 900)
    np.testing.assert_allclose(got["O"], dense.O, rtol=0, atol=1e-5 * np.abs(dense.O).max())


def test_n_at_least_length_is_dense():
    w, x = small(2, 8, 2, 8, 64, [50, 300], "bf16", seed=32)
    g = GpuCase(x, 64, sel_cap=300)
    got = g.step(1, 0)
    ref = oracle_step(x, 64, 1, 0)
    compare(got, ref, x, "bf16", check_tau=True)
    assert np.all(np.isneginf(got["tau"][0])) and np.all(got["count"][0] == 50)


def test_empty_sequences():
    w, x = small(3, 4, 1, 2, 64, [0, 333, 0], "bf16", seed=33, l_max=400)
    g = GpuCase(x, 16)
    g.tau.fill_(0.75)
    got = g.step(2, 0)
    ref = oracle_step(x, 16, 2, 0, tau_in=np.full((3, 4), 0.75))
    compare(got, ref, x, "bf16", check_tau=True)
    assert np.all(got["tau"][[0, 2]] == 0.75)
    # every sequence empty: nothing to stream, zero outputs
    x0 = wl.Inputs(x.q, x.k, x.v, np.zeros(3, np.int32))
    g2 = GpuCase(x0, 16, max_l_kv=0)
    got0 = g2.step(1, 0)
    assert np.all(got0["O"] == 0) and np.all(got0["count"] == 0)


def test_ties_keep_every_equal_logit():
    # every key of the row identical: all logits tie at the threshold, all are kept
    w, x = small(1, 4, 1, 2, 64, [600], "bf16", seed=34)
    x.k[0, 0, :600] = x.k[0, 0, 7]
    g = GpuCase(x, 10, sel_cap=600)
    got = g.step(1, 0)
    assert np.all(got["count"] == 600)
    v = x.v.double().numpy()
    for j in range(4):
        mean = v[0, j // 2, :600].mean(axis=0)
        assert np.abs(got["O"][0, j] - mean).max() <= DERIVED * np.abs(mean).max()


def test_zero_query_keeps_every_key():
    # a query head of zeros: every logit is 0 (the threshold is 0 and every key ties
    # with it), so the head keeps the whole row and averages its value rows; the
    # other heads of the same key head are unaffected
    w, x = small(2, 8, 2, 4, 64, [700, 1500], "bf16", seed=35)
    x.q[1, 3] = 0
    g = GpuCase(x, 16, sel_cap=1500)
    got = g.step(4, 0)
    ref = oracle_step(x, 16, 4, 0)
    compare(got, ref, x, "bf16", check_tau=True)
    assert got["tau"][1, 3] == 0 and got["count"][1, 3] == 1500
    mean = x.v[1, 3 // 2, :1500].double().numpy().mean(axis=0)
    assert np.abs(got["O"][1, 3] - mean).max() <= DERIVED * np.abs(mean).max()
    got1 = g.step(4, 1)                           # the stale zero threshold keeps them again
    assert got1["count"][1, 3] == 1500 and got1["flags"][1, 3] == 0


def test_refresh_with_more_candidates_than_lds():
    # N = l_kv / 5 puts the threshold among the logits between 0.5 and 2 (one top
    # digit of the order key), about 11,000 of a 40,000-key row: more candidates than
    # the finishing select stages in LDS, so it finds their second digit in place
    # first; then a step reusing the refreshed threshold
    w, x = small(2, 4, 1, 2, 64, [40000, 37001], "bf16", seed=37, plant=0.0)
    N = 8000
    g = GpuCase(x, N, sel_cap=40000)
    got = g.step(8, 0)
    ref = oracle_step(x, N, 8, 0)
    compare(got, ref, x, "bf16", check_tau=True)
    got1 = g.step(8, 1)
    ref1 = oracle_step(x, N, 8, 1, tau_in=ref.tau)
    compare(got1, ref1, x, "bf16", check_tau=False)


@pytest.mark.parametrize("hint", ["exact", "above", "below", "far", "zero", "huge", "nan", "minus_inf"])
def test_refresh_result_does_not_depend_on_previous_threshold(hint):
    # a refresh reads the threshold passed in only to guess a window around the new
    # one (a right guess saves a pass over the logits): the exact one and ones 10%
    # above or 8% below it fall inside, the others not; whatever it holds, the
    # refreshed threshold, the kept sets and the outputs are the oracle's
    w, x = small(2, 8, 2, 4, 64, [3000, 1701], "bf16", seed=39)
    N = 24
    ref = oracle_step(x, N, 4, 0)
    tau_in = {"exact": ref.tau, "above": ref.tau * 1.1, "below": ref.tau * 0.92, "far": ref.tau * 1.5,
              "zero": np.zeros_like(ref.tau), "huge": np.full_like(ref.tau, 1e30),
              "nan": np.full_like(ref.tau, np.nan), "minus_inf": np.full_like(ref.tau, -np.inf)}[hint]
    g = GpuCase(x, N)
    got = g.step(4, 0, tau_in=tau_in)
    compare(got, ref, x, "bf16", check_tau=True)
    assert np.all(got["flags"] == 1)


def test_refresh_window_across_a_top_byte_boundary():
    # Thresholds near 2.0, where the top byte of the order key changes: the window
    # guessed around a threshold passed in (about 19% either way) then holds logits of
    # two top bytes, and the finishing select ranks the N-th largest among the
    # candidates of its own byte, by the histogram's rank below the boundary and by
    # the count above the window above it. The thresholds passed in are the exact
    # ones; every row is compared with the oracle, and the rows are checked to fall
    # on both sides of the boundary.
    w, x = small(2, 8, 2, 4, 64, [6000, 5003], "bf16", seed=41, plant=0.0)
    seen = {"below": 0, "above": 0}
    for N in (90, 110, 130, 150, 170):
        ref = oracle_step(x, N, 1, 0)
        g = GpuCase(x, N, sel_cap=4 * N)
        got = g.step(1, 0, tau_in=ref.tau)
        compare(got, ref, x, "bf16", check_tau=True)
        t = ref.tau[np.isfinite(ref.tau)]
        seen["below"] += int(np.sum((t > 2.0 * 2 ** -0.25) & (t < 2.0)))
        seen["above"] += int(np.sum((t >= 2.0) & (t < 2.0 * 2 ** 0.25)))
    assert seen["below"] > 0 and seen["above"] > 0, seen


def test_refresh_window_with_negative_thresholds():
    # N = 3/4 of the row: the thresholds are negative logits; the window around a
    # threshold passed in (the exact one, 5% larger or smaller in magnitude) holds
    # the new one, and the result is the oracle's
    w, x = small(1, 8, 2, 4, 64, [4000], "bf16", seed=42, plant=0.0)
    N = 3000
    ref = oracle_step(x, N, 1, 0)
    assert np.all(ref.tau < 0)
    for f in (1.0, 1.05, 0.95):
        g = GpuCase(x, N, sel_cap=4000)
        got = g.step(1, 0, tau_in=ref.tau * f)
        compare(got, ref, x, "bf16", check_tau=True)


def test_ties_beyond_lds_capacity():
    # 9000 identical keys: all logits of a row are one value, so all 9000 are
    # threshold candidates sharing their second digit too, staged in the row's
    # global buffer; every key ties with the threshold and is kept
    w, x = small(1, 4, 1, 2, 64, [9000], "bf16", seed=38)
    x.k[0, 0, :9000] = x.k[0, 0, 11]
    g = GpuCase(x, 100, sel_cap=9000)
    got = g.step(1, 0)
    ref = oracle_step(x, 100, 1, 0)
    assert np.all(np.abs(got["tau"] - ref.tau) <= 1e-5 * np.abs(ref.tau))
    assert np.all(got["count"] == 9000)
    v = x.v.double().numpy()
    for j in range(4):
        mean = v[0, j // 2, :9000].mean(axis=0)
        assert np.abs(got["O"][0, j] - mean).max() <= DERIVED * np.abs(mean).max()


@pytest.mark.parametrize("scale", [0.05, 2.5])
def test_given_logit_scale(scale):
    # a logit scale other than 1/sqrt(d) (saga_shape.scale): the decode step (refresh
    # and stale) and the dense kernel against the oracle with the same scale
    w, x = small(2, 12, 1, 4, 128, [3000, 777], "bf16", seed=36)
    N = 32
    dev = torch.device("cuda:0")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    l_kv = torch.from_numpy(x.l_kv).to(dev)
    tau = torch.zeros(2, 12, dtype=torch.float32, device=dev)
    cnt = torch.zeros(2, 12, dtype=torch.int32, device=dev)
    idx = torch.full((2, 12, 4 * N), -1, dtype=torch.int32, device=dev)
    q64, k64, v64 = x.f64()
    tau_o = None
    for step in (0, 1):
        out = api.decode_attn(q, k, v, l_kv, tau, N=N, refresh_period=4, step=step, out_dtype=torch.float32,
                              sel_count=cnt, sel_idx=idx, scale=scale)
        torch.cuda.synchronize()
        got = dict(O=out.double().cpu().numpy(), tau=tau.double().cpu().numpy(), count=cnt.cpu().numpy(),
                   idx=idx.cpu().numpy())
        ref = orc.saga_decode_step(q64, k64, v64, x.l_kv, N, 4, step, tau_in=tau_o, scale=scale)
        compare(got, ref, x, "bf16", check_tau=(step == 0))
        tau_o = ref.tau
    dense = api.dense_gqa_attn(q, k, v, l_kv, out_dtype=torch.float32, scale=scale)
    torch.cuda.synchronize()
    ref_d = orc.dense_gqa(q64, k64, v64, x.l_kv, scale=scale)
    got_d = dense.double().cpu().numpy()
    for b in range(2):
        for j in range(12):
            assert np.abs(got_d[b, j] - ref_d[b, j]).max() <= DERIVED * np.abs(ref_d[b, j]).max(), (b, j)


def test_kept_index_export_capacity():
    # sel_cap below the kept count: sel_count is still the whole count, the export holds
    # sel_cap distinct kept indices (any of them), and the output is the whole set's
    w, x = small(2, 12, 1, 4, 128, [4000, 1300], "bf16", seed=37)
    N = 64
    g = GpuCase(x, N, sel_cap=20)
    got = g.step(4, 0)
    ref = oracle_step(x, N, 4, 0)
    compare(got, ref, x, "bf16", check_tau=True, cap_ok=False)
    for b in range(2):
        for j in range(12):
            assert got["count"][b, j] == len(ref.sel[b][j]) >= 20
            e = got["idx"][b, j]
            assert len(set(e.tolist())) == 20 and set(e.tolist()) <= set(ref.sel[b][j].tolist()), (b, j)


# --- the other entry points --------------------------------------------------------

def test_refresh_threshold_entry_point():
    w, x = small(2, 12, 1, 4, 128, [3000, 1200], "bf16", seed=35)
    g = GpuCase(x, 1)
    q64, k64, _ = x.f64()
    for N in (1, 7, 100, 1199, 1200, 5000):
        api.refresh_threshold(g.q, g.k, g.l_kv, g.tau, N=N, max_l_kv=g.max_l_kv, workspace=g.ws)
        torch.cuda.synchronize()
        got = g.tau.double().cpu().numpy()
        want = orc.refresh_threshold(q64, k64, x.l_kv, N)
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(got), fin), N
        assert np.all(got[~fin] == want[~fin])
        assert np.all(np.abs(got[fin] - want[fin]) <= 1e-5 * np.abs(want[fin])), N


def test_stages_equal_decode_step():
    w, x = small(1, 12, 1, 4, 128, [6000], "bf16", seed=36)
    g = GpuCase(x, 64)
    g.step(8, 0)
    ref = g.step(8, 1)
    tau = g.tau.clone()
    out = torch.empty_like(g.out)
    api.qk_select(g.q, g.k, g.l_kv, tau, max_l_kv=g.max_l_kv, workspace=g.ws)
    api.sparse_gather(g.q, g.k, g.v, g.l_kv, tau, N=64, max_l_kv=g.max_l_kv, out=out, workspace=g.ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.double().cpu().numpy(), ref["O"], rtol=0, atol=1e-5 * np.abs(ref["O"]).max())
    # the two kernels of the step, one call each: the same launches as the step itself
    out2 = torch.empty_like(g.out)
    cnt = torch.zeros_like(g.sel_count)
    api.select_gather(g.q, g.k, g.v, g.l_kv, tau, N=64, max_l_kv=g.max_l_kv, workspace=g.ws)
    api.split_combine(g.q, g.k, g.v, g.l_kv, tau, N=64, max_l_kv=g.max_l_kv, out=out2, sel_count=cnt,
                      workspace=g.ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out2.double().cpu().numpy(), ref["O"], rtol=0, atol=1e-6 * np.abs(ref["O"]).max())
    assert np.array_equal(cnt.cpu().numpy(), ref["count"])


DENSE = [
    # B, h_q, h_k, h_v, d, lens, dtype  (h_k == h_v: grouped-query; h_k < h_v: SAGA, full attention)
    (1, 12, 2, 2, 128, [5000], "bf16"),
    (2, 32, 8, 8, 64, [3000, 17], "bf16"),
    (3, 4, 1, 1, 64, [1, 0, 700], "f32"),
    (1, 16, 1, 1, 128, [2049], "f32"),
    (1, 12, 1, 4, 128, [5000], "bf16"),
    (2, 32, 2, 8, 64, [3000, 1], "bf16"),
    (1, 16, 1, 16, 128, [777], "f32"),
]


@pytest.mark.parametrize("case", range(len(DENSE)))
def test_dense_gqa(case):
    B, h_q, h_k, h_v, d, lens, dtype = DENSE[case]
    say(f"dense case {case}: {DENSE[case]}")
    w, x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=40 + case)
    dev = torch.device("cuda:0")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    l_kv = torch.from_numpy(x.l_kv).to(dev)
    out = api.dense_gqa_attn(q, k, v, l_kv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q64, k64, v64 = x.f64()
    ref = orc.dense_gqa(q64, k64, v64, x.l_kv)
    got = out.double().cpu().numpy()
    tol = out_bound(dtype)
    for b in range(B):
        if x.l_kv[b] == 0:
            assert np.all(got[b] == 0)
            continue
        for j in range(h_q):
            s = np.abs(ref[b, j]).max()
            assert np.abs(got[b, j] - ref[b, j]).max() <= tol * s, (b, j)


def test_dense_saga_full_size():
    # SAGA with full attention at the Qwen-shaped 128K layer (h_k=1, h_v=4)
    w = wl.QWEN_128K
    x = wl.generate(w, seed=0)
    dev = torch.device("cuda:0")
    out = api.dense_gqa_attn(x.q.to(dev), x.k.to(dev), x.v.to(dev), torch.from_numpy(x.l_kv).to(dev),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    q64, k64, v64 = x.f64()
    ref = orc.dense_gqa(q64, k64, v64, x.l_kv)
    got = out.double().cpu().numpy()
    err = np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
    assert err.max() <= 2e-3, err.max()


@pytest.mark.parametrize("name", ["llama3.2-1b-shape-l32k", "qwen2.5-1.5b-shape-l128k"])
def test_dense_gqa_full_size(name):
    w0 = wl.WORKLOADS[name]
    w = w0.with_(h_k=w0.dense_h_kv, h_v=w0.dense_h_kv, workload_id=w0.workload_id + 100)
    x = wl.generate(w, seed=0)
    dev = torch.device("cuda:0")
    out = api.dense_gqa_attn(x.q.to(dev), x.k.to(dev), x.v.to(dev), torch.from_numpy(x.l_kv).to(dev),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    q64, k64, v64 = x.f64()
    ref = orc.dense_gqa(q64, k64, v64, x.l_kv)
    got = out.double().cpu().numpy()
    err = np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
    assert err.max() <= 2e-3, err.max()


@pytest.mark.parametrize("case", [
    # B, h_q, h_k, h_v, d, lens, N (a long row with about one kept entry per chunk; a
    # short row whose heads are split over several blocks per chunk; fp32 caches)
    (1, 12, 1, 4, 128, [65536], 256, "bf16"),
    (1, 12, 1, 4, 128, [4096], 2048, "bf16"),
    (2, 8, 2, 4, 64, [3000, 1234], 100, "f32"),
])
def test_repeated_steps_are_bitwise_identical(case):
    # kept entries take fixed slots (each lane's first slot is the sum of the kept
    # counts of the lanes before it) and every sum runs in a fixed order, so the same
    # step on the same inputs gives the same bits every time
    B, h_q, h_k, h_v, d, lens, N, dtype = case
    w, x = small(B, h_q, h_k, h_v, d, lens, dtype, seed=50)
    g = GpuCase(x, N)
    runs = []
    for _ in range(3):
        r0 = g.step(8, 0)
        r1 = g.step(8, 3)
        runs.append((r0, r1))
    for r0, r1 in runs[1:]:
        for got, ref in ((r0, runs[0][0]), (r1, runs[0][1])):
            for key in ("O", "tau", "count", "idx", "flags"):
                assert np.array_equal(got[key], ref[key]), key
    compare(runs[0][0], oracle_step(x, N, 8, 0), x, dtype, check_tau=True)
