"""The Python binding refuses tensors of the wrong size before anything is launched.

The kernels write B*h_q counts and flags, cap kept indices per row, B*d_model layer
outputs and B new lengths; a smaller tensor would be written past its end. Each
case below must raise ValueError, and the tensors the call would have written must
be untouched afterwards (nothing was enqueued).
"""
import pytest
import torch

from sparse_decode_attention_saga_amd import api

DEV = torch.device("cuda:0")
pytestmark = pytest.mark.gpu


def _inputs(B=2, h_q=4, h_k=1, h_v=2, d=64, L=96):
    g = torch.Generator().manual_seed(0)
    q = torch.randn(B, h_q, d, generator=g).to(DEV)
    k = torch.randn(B, h_k, L, d, generator=g).to(DEV)
    v = torch.randn(B, h_v, L, d, generator=g).to(DEV)
    l_kv = torch.full((B,), L, dtype=torch.int32, device=DEV)
    tau = torch.zeros(B, h_q, dtype=torch.float32, device=DEV)
    return q, k, v, l_kv, tau


@pytest.mark.parametrize("bad", ["sel_count", "flags", "sel_idx_rows", "sel_idx_2d", "tau", "l_kv", "out"])
def test_decode_attn_refuses_missized_outputs(bad):
    q, k, v, l_kv, tau = _inputs()
    B, h_q = q.shape[:2]
    kw = dict(sel_count=torch.zeros(B, h_q, dtype=torch.int32, device=DEV),
              flags=torch.zeros(B, h_q, dtype=torch.int32, device=DEV),
              sel_idx=torch.full((B, h_q, 8), -7, dtype=torch.int32, device=DEV),
              out=torch.full((B, h_q, 64), 5.0, device=DEV))
    if bad == "sel_count":
        kw["sel_count"] = torch.zeros(B * h_q - 1, dtype=torch.int32, device=DEV)
    elif bad == "flags":
        kw["flags"] = torch.zeros(B, h_q - 1, dtype=torch.int32, device=DEV)
    elif bad == "sel_idx_rows":
        kw["sel_idx"] = torch.full((B, h_q - 1, 8), -7, dtype=torch.int32, device=DEV)
    elif bad == "sel_idx_2d":
        kw["sel_idx"] = torch.full((B, h_q), -7, dtype=torch.int32, device=DEV)
    elif bad == "tau":
        tau = torch.zeros(B, h_q - 1, dtype=torch.float32, device=DEV)
    elif bad == "l_kv":
        l_kv = torch.full((B + 1,), 96, dtype=torch.int32, device=DEV)
    elif bad == "out":
        kw["out"] = torch.full((B, h_q, 32), 5.0, device=DEV)
    before = {n: t.clone() for n, t in kw.items()}
    with pytest.raises(ValueError):
        api.decode_attn(q, k, v, l_kv, tau, N=8, refresh_period=1, step=0, **kw)
    torch.cuda.synchronize()
    for n, t in kw.items():
        assert torch.equal(t, before[n]), n


def test_decode_attn_accepts_well_sized_outputs():
    q, k, v, l_kv, tau = _inputs()
    B, h_q = q.shape[:2]
    sel_count = torch.zeros(B, h_q, dtype=torch.int32, device=DEV)
    sel_idx = torch.full((B, h_q, 8), -7, dtype=torch.int32, device=DEV)
    api.decode_attn(q, k, v, l_kv, tau, N=8, refresh_period=1, step=0, sel_count=sel_count, sel_idx=sel_idx)
    torch.cuda.synchronize()
    assert torch.all(sel_count == 8)
    assert torch.all(sel_idx >= 0)


def test_decode_layer_refuses_missized_tensors():
    B, h_q, h_k, h_v, d, D, L = 2, 4, 1, 2, 64, 256, 64
    bf = torch.bfloat16
    g = torch.Generator().manual_seed(1)
    x = torch.randn(B, D, generator=g).to(bf).to(DEV)
    w_qkv = (0.05 * torch.randn((h_q + h_k + h_v) * d, D, generator=g)).to(bf).to(DEV)
    w_o = (0.05 * torch.randn(D, h_q * d, generator=g)).to(bf).to(DEV)
    kc = torch.zeros(B, h_k, L, d, dtype=bf, device=DEV)
    vc = torch.zeros(B, h_v, L, d, dtype=bf, device=DEV)
    l_kv = torch.full((B,), 8, dtype=torch.int32, device=DEV)
    l_next = torch.zeros(B, dtype=torch.int32, device=DEV)
    tau = torch.zeros(B, h_q, dtype=torch.float32, device=DEV)
    good = dict(h_q=h_q, N=4, refresh_period=1, step=0, tau=tau, out=torch.empty(B, D, dtype=bf, device=DEV))
    cases = [
        dict(good, out=torch.empty(B, D - 32, dtype=bf, device=DEV)),
        dict(good, tau=torch.zeros(B * h_q - 1, dtype=torch.float32, device=DEV)),
        dict(good, tau=None),
        dict(good, sel_count=torch.zeros(B, dtype=torch.int32, device=DEV)),
        dict(good, flags=torch.zeros(B, h_q + 1, dtype=torch.int32, device=DEV)),
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            api.decode_layer(x, w_qkv, w_o, kc, vc, l_kv, l_next, **kw)
    with pytest.raises(ValueError):
        api.decode_layer(x, w_qkv, w_o, kc, vc, l_kv, torch.zeros(B + 1, dtype=torch.int32, device=DEV), **good)
    with pytest.raises(ValueError):
        api.qkv_append(x, w_qkv, kc, vc, l_kv, l_next, h_q=h_q, q=torch.empty(B, h_q, d // 2, dtype=bf, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(l_next == 0) and torch.all(kc == 0)
