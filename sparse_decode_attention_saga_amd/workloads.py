"""Seeded synthetic inputs for the single-token SAGA decode step.

This module only draws numbers and arranges them into the cache layout. It holds
none of the attention arithmetic, so both the HIP path and the CPU oracle can be
fed from it without sharing any of the method.

Layout (the pages fix none; this is the library's):
  q  [B, h_q, d]            one query row per sequence and query head
  K  [B, h_k, L_max, d]     key cache, token rows d-contiguous
  V  [B, h_v, L_max, d_v]   value cache, token rows d_v-contiguous (d_v = d unless set)
  l_kv [B] int32            valid cache length per sequence (rows >= l_kv[b] are zero)

Recipe (stands in for the model workloads of "More Value per Key: Asymmetric
Sparse Attention for Faster LLM Decoding", Figure 2: Llama 3.2-1B and
Qwen2.5-1.5B decoding at 128K context; no weights or datasets are used):
  * numpy Generator(PCG64) seeded by SeedSequence([workload_id, seed]); nine
    child streams are spawned in a fixed order: q, K, V, plant positions,
    plant head, plant noise, lengths, drift, append.
  * q, K, V are i.i.d. N(0, 1) drawn in float32; bfloat16 workloads are cast
    with round-to-nearest-even, so the oracle and the GPU read identical values.
  * "planted" keys make the score distribution peaked: a planted key of key
    head g is 3 * q_j / |q_j| + 0.1 * N(0, 1), with j a query head drawn
    uniformly from g's group. Its score for head j is about 3 against N(0, 1)
    background scores. Planted positions are single tokens, or non-overlapping
    runs of `run_len` tokens (one head per run).
  * multi-step runs append N(0, 1) K/V rows and drift q as an AR(1) process
    q <- rho*q + sqrt(1 - rho^2)*xi.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

N_STREAMS = 9
(S_Q, S_K, S_V, S_POS, S_HEAD, S_NOISE, S_LEN, S_DRIFT, S_APPEND) = range(N_STREAMS)


@dataclass(frozen=True)
class Workload:
    """One decode-attention workload: head counts, lengths, Atop-N parameters."""

    name: str
    workload_id: int
    batch: int
    h_q: int
    h_k: int
    h_v: int
    d: int
    l_kv: int                      # fixed length, or the upper end of the ragged range
    N: int
    refresh_period: int            # the pages' "n": exact threshold every n steps
    dtype: str                     # "f32" or "bf16"
    plant_frac: float
    run_len: int = 1
    l_kv_min: Optional[int] = None  # set => per-sequence l_kv ~ U{l_kv_min..l_kv}
    dense_h_kv: Optional[int] = None  # head count of the dense GQA baseline
    d_v: Optional[int] = None      # value head dimension when it differs from d

    @property
    def dv(self) -> int:
        return self.d if self.d_v is None else self.d_v

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Workloads, named by what they are. The ids only seed the generators.
TINY = Workload("tiny-fp32-l1024", 1, batch=1, h_q=4, h_k=1, h_v=4, d=64, l_kv=1024,
                N=64, refresh_period=1, dtype="f32", plant_frac=0.01)
LLAMA_32K = Workload("llama3.2-1b-shape-l32k", 2, batch=1, h_q=32, h_k=2, h_v=8, d=64,
                     l_kv=32768, N=256, refresh_period=16, dtype="bf16",
                     plant_frac=0.005, dense_h_kv=8)
QWEN_128K = Workload("qwen2.5-1.5b-shape-l128k", 3, batch=1, h_q=12, h_k=1, h_v=4, d=128,
                     l_kv=131072, N=512, refresh_period=32, dtype="bf16",
                     plant_frac=0.005, dense_h_kv=2)
QWEN_128K_B16 = Workload("qwen2.5-1.5b-shape-l128k-b16", 6, batch=16, h_q=12, h_k=1, h_v=4, d=128,
                         l_kv=131072, N=512, refresh_period=32, dtype="bf16",
                         plant_frac=0.005, dense_h_kv=2)
RAGGED_B8 = Workload("ragged-b8-l16k-128k", 4, batch=8, h_q=32, h_k=2, h_v=8, d=64,
                     l_kv=131072, l_kv_min=16384, N=256, refresh_period=16,
                     dtype="bf16", plant_frac=0.005, run_len=64)
SWEEP = Workload("qwen2.5-1.5b-shape-sweep", 5, batch=1, h_q=12, h_k=1, h_v=4, d=128,
                 l_kv=4096, N=512, refresh_period=8, dtype="bf16", plant_frac=0.005,
                 dense_h_kv=2)
# Key heads of half the dimension, twice as many (the same key bytes per token as
# the Llama- and Qwen-shaped workloads above): the reduced key head dimension that
# the pages compare with fewer key heads (section "Training from Scratch").
SIGMA_LLAMA_32K = Workload("llama3.2-1b-shape-sigma-keys-l32k", 7, batch=1, h_q=32, h_k=4, h_v=8, d=32,
                           d_v=64, l_kv=32768, N=256, refresh_period=16, dtype="bf16", plant_frac=0.005)
SIGMA_QWEN_128K = Workload("qwen2.5-1.5b-shape-sigma-keys-l128k", 8, batch=1, h_q=12, h_k=2, h_v=4, d=64,
                           d_v=128, l_kv=131072, N=512, refresh_period=32, dtype="bf16", plant_frac=0.005)
SWEEP_L = (4096, 16384, 65536, 131072)
SWEEP_N = (128, 512, 2048)
SWEEP_PERIOD = (1, 8, 64)

WORKLOADS = {w.name: w for w in (TINY, LLAMA_32K, QWEN_128K, QWEN_128K_B16, RAGGED_B8, SWEEP,
                                 SIGMA_LLAMA_32K, SIGMA_QWEN_128K)}


def streams(workload_id: int, seed: int) -> list:
    """The nine child generators, always spawned in the same order."""
    children = np.random.SeedSequence([workload_id, seed]).spawn(N_STREAMS)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 numpy -> CPU tensor in `dtype` (bfloat16 by round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


@dataclass
class Inputs:
    """One batch of decode inputs as CPU tensors in the workload dtype."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    l_kv: np.ndarray  # int32 [B]

    def f64(self):
        """The exact values as float64 numpy arrays (every bf16/f32 value is exact in f64)."""
        return (self.q.to(torch.float64).numpy(), self.k.to(torch.float64).numpy(),
                self.v.to(torch.float64).numpy())

    @property
    def l_max(self) -> int:
        return self.k.shape[2]


def draw_lengths(w: Workload, rng_len) -> np.ndarray:
    if w.l_kv_min is None:
        return np.full(w.batch, w.l_kv, dtype=np.int32)
    return rng_len.integers(w.l_kv_min, w.l_kv + 1, size=w.batch).astype(np.int32)


def generate(w: Workload, seed: int = 0, l_max: Optional[int] = None,
             lengths: Optional[Sequence[int]] = None,
             plant_frac: Optional[float] = None) -> Inputs:
    """Draw q, K, V and l_kv for workload `w` following the recipe above.

    `l_max` (default: the workload's largest length) is the cache capacity;
    `lengths` overrides the drawn l_kv; `plant_frac` overrides the planted fraction.
    """
    rs = streams(w.workload_id, seed)
    lens = draw_lengths(w, rs[S_LEN]) if lengths is None else np.asarray(lengths, np.int32)
    if lens.shape != (w.batch,):
        raise ValueError("lengths must have one entry per sequence")
    L_max = int(l_max if l_max is not None else max(int(lens.max()), 1))
    if int(lens.max()) > L_max:
        raise ValueError("l_max is smaller than a sequence length")
    frac = w.plant_frac if plant_frac is None else plant_frac
    B, h_q, h_k, h_v, d, dv = w.batch, w.h_q, w.h_k, w.h_v, w.d, w.dv
    g_k = h_q // h_k

    q = rs[S_Q].standard_normal((B, h_q, d), dtype=np.float32)
    K = np.zeros((B, h_k, L_max, d), dtype=np.float32)
    V = np.zeros((B, h_v, L_max, dv), dtype=np.float32)
    for b in range(B):
        L = int(lens[b])
        for g in range(h_k):
            K[b, g, :L] = rs[S_K].standard_normal((L, d), dtype=np.float32)
        for h in range(h_v):
            V[b, h, :L] = rs[S_V].standard_normal((L, dv), dtype=np.float32)

    qhat = q / np.linalg.norm(q, axis=-1, keepdims=True)
    for b in range(B):
        L = int(lens[b])
        for g in range(h_k):
            if w.run_len == 1:
                n_p = int(round(frac * L))
                if n_p == 0:
                    continue
                pos = rs[S_POS].choice(L, size=n_p, replace=False)
                heads = g * g_k + rs[S_HEAD].integers(0, g_k, size=n_p)
            else:
                n_runs = min(int(round(frac * L / w.run_len)), L // w.run_len)
                if n_runs == 0:
                    continue
                starts = rs[S_POS].choice(L // w.run_len, size=n_runs, replace=False) * w.run_len
                pos = (starts[:, None] + np.arange(w.run_len)[None, :]).reshape(-1)
                heads = np.repeat(g * g_k + rs[S_HEAD].integers(0, g_k, size=n_runs), w.run_len)
            noise = rs[S_NOISE].standard_normal((pos.size, d), dtype=np.float32)
            K[b, g, pos] = 3.0 * qhat[b, heads] + 0.1 * noise

    dt = w.torch_dtype
    return Inputs(to_dtype(q, dt), to_dtype(K, dt), to_dtype(V, dt), lens)


@dataclass
class PagedKV:
    """Paged copies of a K/V cache pair (the layout of the library's paged calls).

    k_pages [num_pages, h_k, P, d] and v_pages [num_pages, h_v, P, d] hold the token
    rows, P = page_tokens per page; table[b, p] is the page of tokens [p*P, (p+1)*P)
    of sequence b. Pages are placed in a seeded random order, with `spare` pool pages
    that no sequence uses; table entries for pages wholly past l_kv[b] are set to
    `stale` (any value: the library never uses them for results).
    """

    k_pages: torch.Tensor
    v_pages: torch.Tensor
    table: torch.Tensor  # int32 [B, max_pages]
    page_tokens: int


def paginate(k: torch.Tensor, v: torch.Tensor, l_kv: np.ndarray, page_tokens: int, seed: int = 0,
             spare: int = 3, stale: int = -1) -> PagedKV:
    """Scatter contiguous caches k [B, h_k, L_max, d], v [B, h_v, L_max, d_v] into pages."""
    B, h_k, L_max, d = k.shape
    P = int(page_tokens)
    max_pages = max(1, -(-L_max // P))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x9A9E, seed])))
    num_pages = B * max_pages + spare
    order = rng.permutation(num_pages).astype(np.int32)
    table = order[:B * max_pages].reshape(B, max_pages).copy()
    kp = torch.zeros((num_pages, h_k, P, d), dtype=k.dtype)
    vp = torch.zeros((num_pages, v.shape[1], P, v.shape[3]), dtype=v.dtype)
    for b in range(B):
        for p in range(max_pages):
            lo, hi = p * P, min((p + 1) * P, L_max)
            kp[table[b, p], :, :hi - lo] = k[b, :, lo:hi]
            vp[table[b, p], :, :hi - lo] = v[b, :, lo:hi]
        used = -(-int(l_kv[b]) // P)
        table[b, used:] = stale
    return PagedKV(kp, vp, torch.from_numpy(table), P)


@dataclass
class LayerInputs:
    """Random-init weights of one attention layer and the new token's hidden state
    (the layout of the library's layer calls), as CPU bfloat16 tensors."""

    x: torch.Tensor       # [B, D]
    w_qkv: torch.Tensor   # [(h_q + h_k + h_v) * d, D]: rows of W_Q^T, then W_K^T, then W_V^T
    w_o: torch.Tensor     # [D, h_q * d]: rows of W_O^T


def layer_inputs(w: Workload, seed: int = 0, d_model: Optional[int] = None, h_k: Optional[int] = None,
                 h_v: Optional[int] = None, exact: bool = False) -> LayerInputs:
    """Weights at the workload's head shape (h_k / h_v override it, e.g. for the dense
    baseline's h_kv heads). D = d_model defaults to h_q * d, the hidden size of both
    models the pages time (Llama 3.2-1B: 32 x 64; Qwen2.5-1.5B: 12 x 128).

    Default: x ~ N(0, 1); weight entries ~ N(0, 1 / fan_in) (fan_in = D for w_qkv,
    h_q d for w_o); all rounded to bfloat16 (nearest even).
    exact=True: x entries in {-1, 0, +1} with at most 255 nonzero entries per row and
    w_qkv entries +-2^-4, so every projection is a multiple of 2^-4 of magnitude below
    16: exact in any fp32 summation order and in bfloat16 (at most 8 significant bits).
    w_o is drawn as in the default."""
    h_k = w.h_k if h_k is None else h_k
    h_v = w.h_v if h_v is None else h_v
    D = w.h_q * w.d if d_model is None else int(d_model)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.workload_id, seed, 0x1A7E])))
    n_qkv = (w.h_q + h_k + h_v) * w.d
    if exact:
        x = np.zeros((w.batch, D), np.float32)
        nnz = min(255, D // 4)
        for b in range(w.batch):
            cols = rng.choice(D, size=nnz, replace=False)
            x[b, cols] = rng.choice(np.array([-1.0, 1.0], np.float32), size=nnz)
        w_qkv = rng.choice(np.array([-1.0, 1.0], np.float32), size=(n_qkv, D)) * np.float32(2.0 ** -4)
    else:
        x = rng.standard_normal((w.batch, D), dtype=np.float32)
        w_qkv = rng.standard_normal((n_qkv, D), dtype=np.float32) / np.float32(np.sqrt(D))
    w_o = rng.standard_normal((D, w.h_q * w.d), dtype=np.float32) / np.float32(np.sqrt(w.h_q * w.d))
    bf = torch.bfloat16
    return LayerInputs(to_dtype(x, bf), to_dtype(w_qkv, bf), to_dtype(w_o, bf))


class DecodeStream:
    """A growing cache for multi-step decode runs: appends rows and drifts q.

    The cache tensors are allocated at `l_max` rows once; `append` writes the
    next rows in place, `drift` replaces q. rho = 0.99 is this library's stand-in
    for the pages' remark that attention shifts only marginally between steps.
    """

    def __init__(self, w: Workload, seed: int, l0: int, l_max: int, rho: float = 0.99,
                 plant_frac: Optional[float] = None):
        self.w = w
        self.rho = rho
        base = generate(w, seed, l_max=l_max, lengths=[l0] * w.batch, plant_frac=plant_frac)
        self.q, self.k, self.v = base.q, base.k, base.v
        self._q32 = base.q.to(torch.float32).numpy().copy()
        self.l_kv = base.l_kv.copy()
        rs = streams(w.workload_id, seed)
        self._drift, self._append = rs[S_DRIFT], rs[S_APPEND]

    def append(self, rows: int = 1) -> None:
        w = self.w
        for b in range(w.batch):
            L = int(self.l_kv[b])
            if L + rows > self.k.shape[2]:
                raise ValueError("cache capacity exceeded")
            kn = self._append.standard_normal((w.h_k, rows, w.d), dtype=np.float32)
            vn = self._append.standard_normal((w.h_v, rows, w.dv), dtype=np.float32)
            self.k[b, :, L:L + rows] = to_dtype(kn, w.torch_dtype)
            self.v[b, :, L:L + rows] = to_dtype(vn, w.torch_dtype)
            self.l_kv[b] = L + rows

    def drift(self) -> None:
        xi = self._drift.standard_normal(self._q32.shape, dtype=np.float32)
        self._q32 = (self.rho * self._q32 + np.sqrt(1.0 - self.rho ** 2) * xi).astype(np.float32)
        self.q = to_dtype(self._q32, self.w.torch_dtype)

    def inputs(self) -> Inputs:
        return Inputs(self.q, self.k, self.v, self.l_kv.copy())


@dataclass
class MergeInputs:
    """Calibration hidden states and a teacher's projections for the key-head merge,
    as CPU bfloat16 tensors in the library's layout (projections transposed: row f
    holds output feature f, head-major)."""

    x: torch.Tensor     # [T, D]
    w_q: torch.Tensor   # [h_q * d, D]
    w_k: torch.Tensor   # [h_k * d, D]


def merge_inputs(tokens: int, d_model: int, h_q: int, h_k: int, d: int, seed: int = 0,
                 twins: Sequence[tuple] = (), twin_noise: float = 0.05) -> MergeInputs:
    """x ~ N(0, 1); weight entries ~ N(0, 1/D) (random-init weights at the model's
    shape); all rounded to bfloat16. `twins` lists key-head pairs (a, b) whose
    projections are made close: head b = head a + twin_noise * N(0, 1/D) (a planted
    pairing)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x3E5E, seed])))
    x = rng.standard_normal((tokens, d_model), dtype=np.float32)
    s = np.float32(1.0 / np.sqrt(d_model))
    w_q = rng.standard_normal((h_q * d, d_model), dtype=np.float32) * s
    w_k = rng.standard_normal((h_k * d, d_model), dtype=np.float32) * s
    for a, b in twins:
        w_k[b * d:(b + 1) * d] = w_k[a * d:(a + 1) * d] + np.float32(twin_noise) * s * \
            rng.standard_normal((d, d_model), dtype=np.float32)
    bf = torch.bfloat16
    return MergeInputs(to_dtype(x, bf), to_dtype(w_q, bf), to_dtype(w_k, bf))
