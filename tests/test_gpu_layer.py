"""The decode layer (eq. (1) projections, cache append, attention, W_O) against the
CPU layer oracle on identical seeded inputs (needs an MI355X).

Tolerances (derived from the arithmetic):
  * products y = x w^T accumulate in fp32 in some order: |y - y_ref| <= g_n sum_i
    |x_i w_i| with g_n = n u / (1 - n u), u = 2^-24, plus half a bf16 spacing
    (2^-8 |y| bounds it) when y is stored as bf16;
  * with `exact` layer inputs every projection is exact in fp32 and in bf16, and
    with keys that are multiples of 1/4 in [-2, 2] every q.k dot product is exact in
    fp32 too; so q, the appended cache rows, the logits' order, the selections and
    the kept counts must equal the oracle's exactly (thresholds within the usual
    1e-5 band: the GPU scales its exact dot products in fp32);
  * the attention output entering W_O is rounded to bf16 on both sides from values
    that differ by the attention's fp32 error (about 1e-6 relative), so an element
    may round one bf16 spacing apart: |y_o - y_ref_o| <= sum_c (2^-7 |O_c| +
    1e-5 max|O|) |W_oc| + the product bound.
"""
import numpy as np
import pytest
import torch

from oracle import layer_oracle as lo
from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import workloads as wl
from tests.parity import BAND, row_scale

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U = 2.0 ** -24


def say(msg):
    print(f"[layer] {msg}", flush=True)


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def product_bound(x, w):
    """Worst-case fp32 summation error of x w^T, elementwise [B, n_out]."""
    n = x.shape[1]
    g = n * U / (1 - n * U)
    return g * (np.abs(x) @ np.abs(w).T)


LINEAR = [
    # B, n_in, n_out, out dtype
    (1, 1536, 2176, torch.float32),
    (3, 64, 100, torch.float32),
    (16, 2048, 2816, torch.bfloat16),
    (17, 1536, 1536, torch.float32),
    (5, 32, 1, torch.float32),
    (2, 4096, 48, torch.bfloat16),
]


@pytest.mark.parametrize("case", range(len(LINEAR)))
def test_linear(case):
    B, n_in, n_out, odt = LINEAR[case]
    say(f"linear {LINEAR[case]}")
    rng = np.random.default_rng(case)
    x = torch.from_numpy(rng.standard_normal((B, n_in), dtype=np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((n_out, n_in), dtype=np.float32) / np.sqrt(n_in)).to(torch.bfloat16)
    y = api.linear(x.to(DEV), w.to(DEV), out_dtype=odt)
    torch.cuda.synchronize()
    x64, w64 = f64(x), f64(w)
    ref = lo.linear(x64, w64)
    tol = product_bound(x64, w64) + 1e-30
    if odt == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(f64(y) - ref)
    assert np.all(err <= tol), float((err / tol).max())


def exact_keys(x):
    """Keys rounded to multiples of 1/4 in [-2, 2] (rows past l_kv stay zero)."""
    x.k = (torch.round(x.k.float().clamp(-2.0, 2.0) * 4.0) / 4.0).to(torch.bfloat16)
    return x


def small_layer(B, lens, l_max, exact, seed, h_q=12, h_k=1, h_v=4, d=128, N=1, period=1):
    w = wl.Workload("layer-small", 300 + seed, batch=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, l_kv=max(max(lens), 1),
                    N=N, refresh_period=period, dtype="bf16", plant_frac=0.0)
    x = wl.generate(w, seed=seed, lengths=lens, l_max=l_max)
    if exact:
        exact_keys(x)
    return w, x, wl.layer_inputs(w, seed=seed, exact=exact)


@pytest.mark.parametrize("exact", [True, False])
def test_qkv_append(exact):
    w, x, li = small_layer(4, [0, 17, 299, 300], 300, exact, seed=1)
    say(f"qkv append exact={exact}")
    k, v = x.k.to(DEV), x.v.to(DEV)
    l_kv = torch.from_numpy(x.l_kv).to(DEV)
    l_next = torch.full_like(l_kv, -1)
    q = api.qkv_append(li.x.to(DEV), li.w_qkv.to(DEV), k, v, l_kv, l_next, h_q=w.h_q)
    torch.cuda.synchronize()
    proj = lo.linear(f64(li.x), f64(li.w_qkv))
    nq, nk = w.h_q * w.d, w.h_k * w.d
    gq, gk, gv = f64(q).reshape(4, nq), f64(k), f64(v)
    assert l_next.cpu().numpy().tolist() == [1, 18, 300, 300]
    ref_k = np.array(f64(x.k))
    ref_v = np.array(f64(x.v))
    for b, L in enumerate(x.l_kv):
        if L < 300:
            ref_k[b, :, L] = proj[b, nq:nq + nk].reshape(w.h_k, w.d)
            ref_v[b, :, L] = proj[b, nq + nk:].reshape(w.h_v, w.d)
    if exact:
        assert np.array_equal(proj, lo.round_bf16(proj))          # the inputs are built for this
        assert np.array_equal(gq, proj[:, :nq])
        assert np.array_equal(gk, ref_k) and np.array_equal(gv, ref_v)
    else:
        # every stored value is the bf16 rounding of an fp32 sum within the product
        # bound of the exact projection: within one bf16 spacing of that interval
        bnd = product_bound(f64(li.x), f64(li.w_qkv))

        def neighbour(got, p, e):
            spacing = np.ldexp(1.0, np.frexp(np.abs(p) + e)[1] - 8)
            return np.all(np.abs(got - p) <= spacing + e)
        assert neighbour(gq, proj[:, :nq], bnd[:, :nq])
        rows = [b for b, L in enumerate(x.l_kv) if L < 300]
        for b in rows:
            L = x.l_kv[b]
            assert neighbour(gk[b, :, L], ref_k[b, :, L], bnd[b, nq:nq + nk].reshape(w.h_k, w.d))
            assert neighbour(gv[b, :, L], ref_v[b, :, L], bnd[b, nq + nk:].reshape(w.h_v, w.d))
        assert np.mean(gq == lo.round_bf16(proj[:, :nq])) > 0.99
        mask = np.ones(gk.shape, bool)
        for b in rows:
            mask[b, :, x.l_kv[b]] = False
        assert np.array_equal(gk[mask], ref_k[mask])                 # no other cache row changed


class GpuLayer:
    def __init__(self, w, x, li, N, max_l_kv, attention, out_dtype=torch.float32):
        self.h_q, self.N, self.attention = w.h_q, N, attention
        self.k, self.v = x.k.to(DEV), x.v.to(DEV)
        self.l_kv = torch.from_numpy(np.asarray(x.l_kv, np.int32)).to(DEV)
        self.l_next = torch.zeros_like(self.l_kv)
        self.w_qkv, self.w_o = li.w_qkv.to(DEV), li.w_o.to(DEV)
        self.tau = torch.zeros(w.batch, w.h_q, dtype=torch.float32, device=DEV)
        self.count = torch.zeros(w.batch, w.h_q, dtype=torch.int32, device=DEV)
        self.flags = torch.zeros(w.batch, w.h_q, dtype=torch.int32, device=DEV)
        self.max_l_kv = max_l_kv
        L = api.layer_desc(li.x, self.k, self.v, w.h_q, out_dtype)
        self.ws = api.LayerWorkspace(L, N, max_l_kv, DEV)
        self.out_dtype = out_dtype

    def step(self, xin, period, step):
        y = api.decode_layer(xin.to(DEV), self.w_qkv, self.w_o, self.k, self.v, self.l_kv, self.l_next,
                             h_q=self.h_q, attention=self.attention, N=self.N, refresh_period=period, step=step,
                             tau=self.tau, max_l_kv=self.max_l_kv, out_dtype=self.out_dtype, sel_count=self.count,
                             flags=self.flags, workspace=self.ws)
        torch.cuda.synchronize()
        res = dict(y=f64(y), tau=f64(self.tau), count=self.count.cpu().numpy(), flags=self.flags.cpu().numpy(),
                   l_next=self.l_next.cpu().numpy(), K=self.k, V=self.v)
        self.l_kv.copy_(self.l_next)                       # the next token sees this one
        return res


def check_layer(got, ref, li_w_o, where):
    assert np.array_equal(got["l_next"], ref.l_next), where
    w_o = f64(li_w_o)
    O = ref.O.reshape(ref.O.shape[0], -1)
    scale_o = np.abs(O).max(axis=1, keepdims=True)
    bound = (2.0 ** -7 * np.abs(O) + 1e-5 * scale_o) @ np.abs(w_o).T
    bound = bound + product_bound(lo.round_bf16(O), w_o) + 1e-30
    err = np.abs(got["y"] - ref.y)
    assert np.all(err <= bound), f"{where}: y error {float((err / bound).max()):.2f} x the bound"


@pytest.mark.parametrize("attention", ["atopn", "dense"])
def test_decode_layer_exact_inputs(attention):
    B, lens, l_max, N = 2, [4000, 1234], 5000, 64
    w, x, li = small_layer(B, lens, l_max, True, seed=2, N=N, period=4)
    say(f"layer {attention} B={B} lens={lens}")
    mode = api.ATTN_ATOPN if attention == "atopn" else api.ATTN_DENSE
    g = GpuLayer(w, x, li, N, l_max, mode)
    K, V, l_kv, tau = f64(x.k), f64(x.v), np.asarray(x.l_kv), None
    x2 = wl.layer_inputs(w, seed=3, exact=True).x          # the next token's hidden state
    for step, xin in ((0, li.x), (1, x2)):
        got = g.step(xin, 4, step)
        ref = lo.decode_layer(f64(xin), f64(li.w_qkv), f64(li.w_o), K, V, l_kv, w.h_q, attention, N=N,
                              refresh_period=4, step=step, tau_in=tau)
        where = f"step {step}"
        assert np.array_equal(f64(got["K"]), ref.K) and np.array_equal(f64(got["V"]), ref.V), where
        if attention == "atopn":
            r = ref.attn
            for b in range(B):
                for j in range(w.h_q):
                    t_o, t_g = r.tau[b, j], got["tau"][b, j]
                    rs = row_scale(r.logits[b][j])
                    assert abs(t_g - t_o) <= BAND * max(abs(t_o), rs), (where, b, j, t_g, t_o)
                    assert got["count"][b, j] == r.sel[b][j].size, (where, b, j)
            assert np.array_equal(got["flags"], np.where(r.refreshed, 1, 0) | np.where(r.fallback, 2, 0))
            tau = r.tau
        check_layer(got, ref, li.w_o, where)
        K, V, l_kv = ref.K, ref.V, ref.l_next


def test_layer_equals_its_parts():
    # normal weights: the layer call is the three library calls it is made of
    B, lens, l_max, N = 3, [2000, 77, 3999], 4000, 32
    w, x, li = small_layer(B, lens, l_max, False, seed=4, N=N, period=8)
    g = GpuLayer(w, x, li, N, l_max, api.ATTN_ATOPN)
    k2, v2 = x.k.to(DEV), x.v.to(DEV)
    l_kv = torch.from_numpy(x.l_kv).to(DEV)
    l_next = torch.zeros_like(l_kv)
    got = g.step(li.x, 8, 0)
    q = api.qkv_append(li.x.to(DEV), li.w_qkv.to(DEV), k2, v2, l_kv, l_next, h_q=w.h_q)
    tau = torch.zeros(B, w.h_q, dtype=torch.float32, device=DEV)
    cnt = torch.zeros(B, w.h_q, dtype=torch.int32, device=DEV)
    o = api.decode_attn(q, k2, v2, l_next, tau, N=N, refresh_period=8, step=0, max_l_kv=l_max,
                        out_dtype=torch.bfloat16, sel_count=cnt)
    y = api.linear(o.reshape(B, -1), li.w_o.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(g.k, k2) and torch.equal(g.v, v2)
    assert np.array_equal(got["tau"], f64(tau)) and np.array_equal(got["count"], cnt.cpu().numpy())
    # the attention outputs may differ by the order of their sums before their bf16 rounding
    err = np.abs(got["y"] - f64(y)).max() / np.abs(f64(y)).max()
    assert err <= 2.0 ** -6, err


def test_decode_layer_full_size():
    # the Qwen-shaped layer at 128K (131071 cached rows + the new token), Atop-N
    w = wl.QWEN_128K
    x = exact_keys(wl.generate(w, seed=0, lengths=[w.l_kv - 1], l_max=w.l_kv))
    li = wl.layer_inputs(w, seed=0, exact=True)
    say(f"{w.name} layer, D={li.x.shape[1]}")
    g = GpuLayer(w, x, li, w.N, w.l_kv, api.ATTN_ATOPN)
    got = g.step(li.x, w.refresh_period, 0)
    ref = lo.decode_layer(f64(li.x), f64(li.w_qkv), f64(li.w_o), f64(x.k), f64(x.v), x.l_kv, w.h_q, "atopn",
                          N=w.N, refresh_period=w.refresh_period, step=0)
    assert got["l_next"].tolist() == [w.l_kv]
    for j in range(w.h_q):
        assert got["count"][0, j] == ref.attn.sel[0][j].size
    check_layer(got, ref, li.w_o, "full size")
