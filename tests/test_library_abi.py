"""The C-ABI library loads, exports every function include/saga.h declares, and
rejects bad arguments on the host before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_decode_attention_saga_amd import api
from sparse_decode_attention_saga_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "saga.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build_mod.LIB_PATH):
        build_mod.build()
    return api.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(saga_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(api.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in enumerate(["SAGA_OK", "SAGA_ERR_NULL", "SAGA_ERR_SHAPE", "SAGA_ERR_UNSUPPORTED",
                                 "SAGA_ERR_WORKSPACE", "SAGA_ERR_HIP"]):
        assert api.status_str(code) == name
    assert api.status_str(77) == "SAGA_ERR_UNKNOWN"


def shape(**kw):
    d = dict(batch=1, h_q=12, h_k=1, h_v=4, d=128, d_v=0, l_max=131072, dtype=api.BF16, out_dtype=api.BF16,
             scale=0.0)
    d.update(kw)
    return api.SagaShape(**d)


def test_gather_form(lib):
    """Where the step gathers the kept value rows: late (in the combining kernel) for
    value rows of at least 256 bytes, rows of at most 512 chunks, a select kernel of at
    least 512 blocks and a head keeping about CH N / l_kv <= 1 entry per chunk of CH keys
    (<= 2 with 2048 blocks or more); early (in the select kernel) otherwise."""
    def form(N, L, **kw):
        return lib.saga_gather_form(ctypes.byref(shape(**kw)), N, L)
    assert form(512, 131072) == 1                       # Qwen-shaped 128K: 256-key chunks, ~1 kept each
    assert form(512, 131072, batch=16) == 1             # 16 such sequences: 512-key chunks, 4096 blocks
    assert form(512, 131072, d=64, d_v=128) == 0        # 64-wide keys: 512-key chunks, 256 blocks
    assert form(512, 131072, h_k=2, d=64, d_v=128) == 0  # two such key heads: 512 blocks, 2 kept per chunk
    assert form(512, 131072, h_k=2, h_v=2) == 0         # GQA heads (2 key heads of 128): the same
    assert form(2048, 131072) == 0                      # 4 kept per chunk
    assert form(512, 131072, d=64, dtype=api.F32) == 1  # fp32 rows of 64: 256 bytes
    assert form(256, 32768, h_q=32, h_k=2, h_v=8, d=64) == 0  # Llama-shaped 32K: 128-byte value rows
    assert form(2048, 4096) == 0                        # dense selections: 64 kept per 128-key chunk
    assert form(512, 16384) == 0                        # 4 kept per chunk
    assert form(512, 1 << 20, l_max=1 << 20) == 0       # 2048 chunks per row
    assert form(512, 0) == 0                            # nothing cached: the early form's zero rows
    assert form(0, 1024) == -1 and form(8, 1 << 20) == -1 and form(8, 1024, h_k=5) == -1


def test_workspace_bytes(lib):
    s = shape()
    n = lib.saga_workspace_bytes(ctypes.byref(s), 512, 131072)
    # at least the fp32 logits, kept indices and kept logits of every row
    assert n >= 3 * 12 * 131072 * 4
    assert lib.saga_workspace_bytes(ctypes.byref(s), 512, 4096) < n
    assert lib.saga_workspace_bytes(ctypes.byref(shape(h_k=5)), 512, 1024) == 0
    assert lib.saga_workspace_bytes(ctypes.byref(shape(d=96)), 512, 1024) == 0
    assert lib.saga_workspace_bytes(ctypes.byref(s), 0, 1024) == 0
    assert lib.saga_workspace_bytes(ctypes.byref(s), 8, 131073) == 0


@pytest.mark.parametrize("kw", [dict(), dict(batch=3), dict(h_q=32, h_k=2, h_v=8, d=64), dict(dtype=api.F32, out_dtype=api.F32),
                                dict(h_q=32, h_k=4, h_v=8, d=32, d_v=64)])
def test_workspace_grows_with_context(lib, kw):
    # the launch picks its chunk width from max_l_kv (narrower chunks, more records
    # below some lengths); a workspace sized for a length serves every shorter one
    s = shape(**kw)
    lengths = sorted({1, 127, 128, 129, 4095, 4096, 16384, 32767, 32768, 65535, 65536, 65537, 98304, 130816,
                      131071, 131072} | {131072 * i // 97 for i in range(1, 97)})
    sizes = [lib.saga_workspace_bytes(ctypes.byref(s), 512, L) for L in lengths]
    assert all(n > 0 for n in sizes)
    assert all(a <= b for a, b in zip(sizes, sizes[1:])), list(zip(lengths, sizes))
    assert lib.saga_workspace_bytes(None, 8, 16) == 0


def test_head_dimension_pairs(lib):
    """Built (d, d_v): equal dimensions 64 and 128, and the reduced key dimensions
    (32, 64) and, for bf16, (64, 128); d_v = 0 means d_v = d."""
    def ok(**kw):
        return lib.saga_workspace_bytes(ctypes.byref(shape(**kw)), 64, 4096) > 0
    assert ok(d=128, d_v=0) and ok(d=128, d_v=128) and ok(d=64, d_v=0)
    assert ok(d=32, d_v=64) and ok(d=32, d_v=64, dtype=api.F32, out_dtype=api.F32)
    assert ok(d=64, d_v=128) and not ok(d=64, d_v=128, dtype=api.F32, out_dtype=api.F32)
    assert not ok(d=32, d_v=0) and not ok(d=128, d_v=64) and not ok(d=64, d_v=-1) and not ok(d=32, d_v=128)
    small = lib.saga_workspace_bytes(ctypes.byref(shape(d=64, d_v=64)), 64, 4096)
    assert lib.saga_workspace_bytes(ctypes.byref(shape(d=64, d_v=128)), 64, 4096) > small


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def decode(lib, s, N=8, period=4, step=1, ws_bytes=1 << 40, max_l=1024, tau=FAKE, sel_idx=None, cap=0):
    return lib.saga_decode_attn(None if s is None else ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, max_l, N,
                                period, step, tau, FAKE, None, sel_idx, cap, None, FAKE, ws_bytes, None)


def decode_noalloc(lib, s, N=8, period=4, step=1, max_l=1024, tau=FAKE, sel_idx=None, cap=0):
    return lib.saga_decode_attn_noalloc(None if s is None else ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, max_l, N,
                                        period, step, tau, FAKE, None, sel_idx, cap, None, None)


def test_noalloc_rejects_bad_arguments_before_touching_the_gpu(lib):
    # the same checks as saga_decode_attn, and a step that needs more scratch than
    # SAGA_NOALLOC_SCRATCH_BYTES is refused with SAGA_ERR_WORKSPACE
    assert decode_noalloc(lib, None) == api.ERR_NULL
    assert decode_noalloc(lib, shape(), tau=None) == api.ERR_NULL
    assert decode_noalloc(lib, shape(h_k=5)) == api.ERR_SHAPE
    assert decode_noalloc(lib, shape(batch=0)) == api.ERR_SHAPE
    assert decode_noalloc(lib, shape(), N=0) == api.ERR_SHAPE
    assert decode_noalloc(lib, shape(), period=0) == api.ERR_SHAPE
    assert decode_noalloc(lib, shape(), step=-1) == api.ERR_SHAPE
    assert decode_noalloc(lib, shape(), max_l=131073) == api.ERR_SHAPE
    assert decode_noalloc(lib, shape(), sel_idx=FAKE, cap=0) == api.ERR_SHAPE
    assert decode_noalloc(lib, shape(d=96)) == api.ERR_UNSUPPORTED
    big = shape(batch=4)
    assert lib.saga_workspace_bytes(ctypes.byref(big), 512, 131072) > api.NOALLOC_SCRATCH_BYTES
    assert decode_noalloc(lib, big, N=512, max_l=131072) == api.ERR_WORKSPACE
    # the header's scratch size and the binding's agree
    text = open(HEADER).read()
    m = re.search(r"#define SAGA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == api.NOALLOC_SCRATCH_BYTES


def test_decode_rejects_bad_arguments(lib):
    assert decode(lib, None) == api.ERR_NULL
    assert decode(lib, shape(), tau=None) == api.ERR_NULL
    assert decode(lib, shape(h_k=5)) == api.ERR_SHAPE
    assert decode(lib, shape(h_v=7)) == api.ERR_SHAPE
    assert decode(lib, shape(batch=0)) == api.ERR_SHAPE
    assert decode(lib, shape(scale=-1.0)) == api.ERR_SHAPE
    assert decode(lib, shape(), N=0) == api.ERR_SHAPE
    assert decode(lib, shape(), period=0) == api.ERR_SHAPE
    assert decode(lib, shape(), step=-1) == api.ERR_SHAPE
    assert decode(lib, shape(), max_l=131073) == api.ERR_SHAPE
    assert decode(lib, shape(), max_l=-1) == api.ERR_SHAPE
    assert decode(lib, shape(), sel_idx=FAKE, cap=0) == api.ERR_SHAPE
    assert decode(lib, shape(d=96)) == api.ERR_UNSUPPORTED
    assert decode(lib, shape(dtype=7)) == api.ERR_UNSUPPORTED
    assert decode(lib, shape(out_dtype=2)) == api.ERR_UNSUPPORTED
    # more (sequence, query head) rows than the kernels index: refused before any work
    assert decode(lib, shape(batch=65535, h_q=512, h_k=1, h_v=1)) == api.ERR_UNSUPPORTED
    assert lib.saga_workspace_bytes(ctypes.byref(shape(batch=65535, h_q=512, h_k=1, h_v=1)), 8, 1024) == 0
    assert decode(lib, shape(), ws_bytes=1024) == api.ERR_WORKSPACE


def test_other_entry_points_reject_bad_arguments(lib):
    s = shape()
    big = 1 << 40
    assert lib.saga_refresh_threshold(ctypes.byref(s), FAKE, FAKE, FAKE, 1024, 0, FAKE, FAKE, big, None) == api.ERR_SHAPE
    assert lib.saga_refresh_threshold(ctypes.byref(s), FAKE, FAKE, FAKE, 1024, 4, FAKE, FAKE, 16, None) == api.ERR_WORKSPACE
    assert lib.saga_qk_select(ctypes.byref(s), FAKE, None, FAKE, 1024, FAKE, FAKE, big, None) == api.ERR_NULL
    assert lib.saga_sparse_gather(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1024, 8, FAKE, None, None, None, 0,
                                  None, FAKE, big, None) == api.ERR_NULL
    assert lib.saga_select_gather(ctypes.byref(s), FAKE, FAKE, None, FAKE, 1024, 8, FAKE, FAKE, big, None) == api.ERR_NULL
    assert lib.saga_select_gather(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1024, 0, FAKE, FAKE, big,
                                  None) == api.ERR_SHAPE
    assert lib.saga_select_gather(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1024, 8, FAKE, FAKE, 16, None) == api.ERR_WORKSPACE
    assert lib.saga_split_combine(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1024, 0, FAKE, FAKE, None, None, 0,
                                  None, FAKE, big, None) == api.ERR_SHAPE
    assert lib.saga_split_combine(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1024, 8, FAKE, FAKE, None, FAKE, 0,
                                  None, FAKE, big, None) == api.ERR_SHAPE
    # dense attention: the query heads of a value head must share a key head (h_k | h_v),
    # at most 16 query heads per value head
    more_keys = shape(h_q=8, h_k=4, h_v=2)
    assert lib.saga_dense_gqa_attn(ctypes.byref(more_keys), FAKE, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, big,
                                   None) == api.ERR_UNSUPPORTED
    wide = shape(h_q=32, h_k=1, h_v=1)
    assert lib.saga_dense_gqa_attn(ctypes.byref(wide), FAKE, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, big, None) == api.ERR_UNSUPPORTED
    assert lib.saga_dense_gqa_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1024, None, FAKE, big, None) == api.ERR_NULL
    assert lib.saga_workspace_init(None, 16, None) == api.ERR_NULL


def pages(table=FAKE, max_pages=64, page_tokens=16, num_pages=64):
    return api.SagaPages(table.value if table is not None else None, max_pages, page_tokens, num_pages)


def decode_paged(lib, pg, max_l=1024, s=None):
    s = shape() if s is None else s
    return lib.saga_decode_attn_paged(ctypes.byref(s), None if pg is None else ctypes.byref(pg), FAKE, FAKE,
                                      FAKE, FAKE, max_l, 8, 4, 1, FAKE, FAKE, None, None, 0, None, FAKE,
                                      1 << 40, None)


def test_paged_entry_points_reject_bad_page_descriptors(lib):
    assert decode_paged(lib, None) == api.ERR_NULL
    assert decode_paged(lib, pages(table=None)) == api.ERR_NULL
    assert decode_paged(lib, pages(page_tokens=8)) == api.ERR_SHAPE          # below one 16-key tile
    assert decode_paged(lib, pages(page_tokens=48)) == api.ERR_SHAPE         # not a power of two
    assert decode_paged(lib, pages(max_pages=63)) == api.ERR_SHAPE           # 63 * 16 < 1024 tokens
    assert decode_paged(lib, pages(num_pages=0)) == api.ERR_SHAPE
    assert decode_paged(lib, pages(), s=shape(h_k=5)) == api.ERR_SHAPE       # shape checks still apply
    assert decode_paged(lib, pages(), max_l=131073) == api.ERR_SHAPE
    pg = pages(page_tokens=32)
    assert lib.saga_dense_gqa_attn_paged(ctypes.byref(shape()), ctypes.byref(pg), FAKE, FAKE, FAKE, FAKE, 1024,
                                         None, FAKE, 1 << 40, None) == api.ERR_NULL
    assert lib.saga_dense_gqa_attn_paged(ctypes.byref(shape()), ctypes.byref(pages(max_pages=1)), FAKE, FAKE,
                                         FAKE, FAKE, 1024, FAKE, FAKE, 1 << 40, None) == api.ERR_SHAPE


def layer(d_model=1536, **kw):
    return api.SagaLayer(shape(l_max=4096, **kw), d_model)


def test_layer_entry_points_reject_bad_arguments(lib):
    big = 1 << 40
    L = layer()
    assert lib.saga_layer_workspace_bytes(ctypes.byref(L), 512, 4096) > lib.saga_workspace_bytes(
        ctypes.byref(L.attn), 512, 4096)
    assert lib.saga_layer_workspace_bytes(ctypes.byref(layer(d_model=100)), 512, 4096) == 0
    assert lib.saga_layer_workspace_bytes(ctypes.byref(layer(dtype=api.F32)), 512, 4096) == 0
    assert lib.saga_linear(1, 1536, 10, FAKE, FAKE, None, api.F32, None) == api.ERR_NULL
    assert lib.saga_linear(1, 100, 10, FAKE, FAKE, FAKE, api.F32, None) == api.ERR_SHAPE   # n_in % 32
    assert lib.saga_linear(0, 64, 10, FAKE, FAKE, FAKE, api.F32, None) == api.ERR_SHAPE
    assert lib.saga_linear(1, 64, 10, FAKE, FAKE, FAKE, 7, None) == api.ERR_UNSUPPORTED
    assert lib.saga_linear(1, 1 << 20, 10, FAKE, FAKE, FAKE, api.F32, None) == api.ERR_UNSUPPORTED
    assert lib.saga_qkv_append(ctypes.byref(L), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == api.ERR_NULL
    assert lib.saga_qkv_append(ctypes.byref(L), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == api.ERR_SHAPE
    assert lib.saga_qkv_append(ctypes.byref(layer(dtype=api.F32)), FAKE, FAKE, FAKE, FAKE, FAKE,
                               ctypes.c_void_p(0x2000), FAKE, None) == api.ERR_UNSUPPORTED

    def dl(L, attention=api.ATTN_ATOPN, tau=FAKE, max_l=4096, N=8, period=4, step=1, ws=big, l_next=None):
        return lib.saga_decode_layer(ctypes.byref(L), attention, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     l_next or ctypes.c_void_p(0x2000), max_l, N, period, step, tau, FAKE, None,
                                     None, FAKE, ws, None)
    assert dl(L, tau=None) == api.ERR_NULL
    assert dl(L, attention=5) == api.ERR_UNSUPPORTED
    assert dl(L, max_l=4097) == api.ERR_SHAPE
    assert dl(L, N=0) == api.ERR_SHAPE
    assert dl(L, period=0) == api.ERR_SHAPE
    assert dl(L, l_next=FAKE) == api.ERR_SHAPE            # l_kv and l_kv_next alias
    assert dl(L, ws=1024) == api.ERR_WORKSPACE
    assert dl(layer(d_model=48)) == api.ERR_SHAPE
    assert dl(layer(h_q=8, h_k=4, h_v=2), attention=api.ATTN_DENSE, tau=None) == api.ERR_UNSUPPORTED


def test_paginate_places_every_token_row():
    import numpy as np
    import torch
    from sparse_decode_attention_saga_amd import workloads as wl
    w = wl.Workload("paginate", 7, batch=3, h_q=4, h_k=2, h_v=4, d=64, l_kv=300, N=4, refresh_period=1,
                    dtype="bf16", plant_frac=0.0)
    x = wl.generate(w, seed=1, lengths=[300, 17, 0], l_max=300)
    pk = wl.paginate(x.k, x.v, x.l_kv, 64, seed=2, stale=-9)
    assert pk.k_pages.shape == (3 * 5 + 3, 2, 64, 64) and pk.v_pages.shape == (18, 4, 64, 64)
    tab = pk.table.numpy()
    assert np.all(tab[1, 1:] == -9) and np.all(tab[2] == -9)
    used = tab[tab >= 0]
    assert len(set(used.tolist())) == used.size                                # no page shared
    for b in range(3):
        for i in range(int(x.l_kv[b])):
            pg = tab[b, i // 64]
            assert torch.equal(pk.k_pages[pg, :, i % 64], x.k[b, :, i])
            assert torch.equal(pk.v_pages[pg, :, i % 64], x.v[b, :, i])


def test_binding_requires_gpu_tensors(lib):
    import torch
    q = torch.zeros(1, 4, 64)
    k = torch.zeros(1, 1, 16, 64)
    with pytest.raises(ValueError):
        api.decode_attn(q, k, k, torch.zeros(1, dtype=torch.int32), torch.zeros(1, 4), N=4, refresh_period=1, step=0)


def merge_shape(**kw):
    d = dict(tokens=4096, d_model=2048, h_q=32, h_k=8, d=64)
    d.update(kw)
    return api.SagaMergeShape(**d)


def test_merge_workspace_bytes(lib):
    s = merge_shape()
    n = lib.saga_merge_workspace_bytes(ctypes.byref(s))
    # at least the fp32 queries and keys of every calibration token
    assert n >= 4096 * (32 + 8) * 64 * 4
    assert lib.saga_merge_workspace_bytes(ctypes.byref(merge_shape(h_k=7, h_q=28))) == 0   # odd head count
    assert lib.saga_merge_workspace_bytes(ctypes.byref(merge_shape(h_k=18, h_q=36))) == 0  # more than 16 heads
    assert lib.saga_merge_workspace_bytes(ctypes.byref(merge_shape(d=96))) == 0
    assert lib.saga_merge_workspace_bytes(ctypes.byref(merge_shape(d_model=100))) == 0
    assert lib.saga_merge_workspace_bytes(ctypes.byref(merge_shape(h_q=30))) == 0         # h_k must divide h_q
    assert lib.saga_merge_workspace_bytes(ctypes.byref(merge_shape(d=128, h_k=2, h_q=12, d_model=1536))) > 0
    assert lib.saga_merge_workspace_bytes(None) == 0


@pytest.mark.parametrize("n,seed", [(2, 0), (4, 1), (6, 2), (8, 3), (8, 4), (10, 5)])
def test_host_pairing_equals_oracle_matching(lib, n, seed):
    # Theorem 4.2's matching in the library's host code against the oracle's
    # enumeration of every perfect matching (no device work is involved)
    from oracle import convert_oracle as cv
    rng = np.random.default_rng(seed)
    w = rng.random((n, n)).astype(np.float32)
    w = w + w.T
    partner, total = api.min_weight_pairing(w)
    pairs, best = cv.min_weight_perfect_matching(w.astype(np.float64))
    assert sorted((a, b) for a, b in enumerate(partner) if a < b) == pairs
    assert abs(total - best) <= 1e-6 * best
    for a in range(n):
        assert partner[partner[a]] == a and partner[a] != a


def test_host_pairing_rejects_bad_input(lib):
    w = np.ones((4, 4), np.float32)
    part = (ctypes.c_int32 * 4)()
    assert lib.saga_min_weight_pairing(3, w.ctypes.data, part, None) == api.ERR_SHAPE
    assert lib.saga_min_weight_pairing(18, w.ctypes.data, part, None) == api.ERR_SHAPE
    assert lib.saga_min_weight_pairing(4, None, part, None) == api.ERR_NULL
    w[1, 2] = np.nan
    assert lib.saga_min_weight_pairing(4, w.ctypes.data, part, None) == api.ERR_SHAPE
    w[1, 2] = 1.0
    w[3, 3] = np.nan          # the diagonal is ignored
    assert lib.saga_min_weight_pairing(4, w.ctypes.data, part, None) == api.OK


def test_host_pairing_sixteen_heads_planted(lib):
    # 16 heads (the largest merge; 2027025 perfect matchings): a planted matching of
    # weight 0.01 per pair against weights >= 1 elsewhere is the unique optimum
    rng = np.random.default_rng(7)
    n = 16
    perm = rng.permutation(n)
    w = (1.0 + rng.random((n, n))).astype(np.float32)
    w = w + w.T
    planted = sorted(tuple(sorted((int(perm[2 * i]), int(perm[2 * i + 1])))) for i in range(n // 2))
    for a, b in planted:
        w[a, b] = w[b, a] = 0.01
    partner, total = api.min_weight_pairing(w)
    assert sorted((a, b) for a, b in enumerate(partner) if a < b) == planted
    assert abs(total - 0.08) <= 1e-6
