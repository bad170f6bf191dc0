"""CPU oracle of the decode layer around the SAGA + Atop-N attention step.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the entry module and the
CPU-baseline leg of the benchmark may import this module. The library and its
binding never do, and this module shares no code with them.

Plain float64 numpy, as in saga_oracle (whose attention step this module calls).
What it follows (the paper "More Value per Key: Asymmetric Sparse Attention for
Faster LLM Decoding", summary page picx.dev DRD92V):
  * section "Attention Mechanism Formalization", eq. (1): Q = X W_Q, K = X W_K,
    V = X W_V, for the one new token of each sequence;
  * section "SAGA Architecture": W_K has h_k heads and W_V has h_v heads;
  * the attention step of saga_oracle (Atop-N, or dense eq. (2)-(4)) over the cache
    with the new token's key and value rows appended;
  * the output projection W_O of multi-head attention applied to the attention
    output of all query heads, concatenated head by head.

Readings taken where the pages are silent:
  * weights are stored as in the library: w_qkv [(h_q + h_k + h_v) d, D] holds the
    rows of W_Q^T, then W_K^T, then W_V^T (head-major features), w_o [D, h_q d] the
    rows of W_O^T;
  * the caches hold bfloat16, so the new key and value rows are their projections
    rounded to the nearest bfloat16 (ties to even); q is rounded the same way, as
    the attention step takes q in the cache's type, and so is the attention output
    entering W_O (the layer's activations are bfloat16);
  * the new rows go to row l_kv[b] of every head, and the attention runs over
    l_kv[b] + 1 rows; a full cache (l_kv[b] == l_max) gets no row;
  * no normalisation, rotary embedding, bias or residual (the pages give none).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from oracle import saga_oracle as so


def round_bf16(x) -> np.ndarray:
    """The nearest bfloat16 value (8 significant bits) of each entry, ties to even,
    as float64. For values inside bfloat16's normal range."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                 # x = m * 2**e with 0.5 <= |m| < 1 (m = 0 for x = 0)
    return np.ldexp(np.rint(m * 256.0), e - 8)   # np.rint rounds halves to even


def linear(x, w) -> np.ndarray:
    """y = x w^T: x [B, n_in], w [n_out, n_in] (row o of w gives output o)."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


@dataclass
class LayerResult:
    y: np.ndarray           # [B, D] layer output
    q: np.ndarray           # [B, h_q, d] bf16-rounded query rows
    K: np.ndarray           # [B, h_k, l_max, d] cache after the append
    V: np.ndarray           # [B, h_v, l_max, d]
    l_next: np.ndarray      # [B] cached rows after the append
    O: np.ndarray           # [B, h_q, d] attention output (before its bf16 rounding)
    attn: Optional[so.DecodeResult]   # the Atop-N step's result (None for dense)


def decode_layer(x, w_qkv, w_o, K, V, l_kv, h_q: int, attention: str = "atopn", N: int = 1,
                 refresh_period: int = 1, step: int = 0, tau_in=None, scale: Optional[float] = None) -> LayerResult:
    """One decode layer for the new token x [B, D] over caches K [B, h_k, l_max, d],
    V [B, h_v, l_max, d] holding l_kv[b] rows. attention: "atopn" or "dense"."""
    x = np.asarray(x, np.float64)
    B = x.shape[0]
    h_k, l_max, d = K.shape[1], K.shape[2], K.shape[3]
    h_v = V.shape[1]
    proj = linear(x, w_qkv)                                   # eq. (1), all three at once
    nq, nk = h_q * d, h_k * d
    q = round_bf16(proj[:, :nq]).reshape(B, h_q, d)
    k_new = round_bf16(proj[:, nq:nq + nk]).reshape(B, h_k, d)
    v_new = round_bf16(proj[:, nq + nk:]).reshape(B, h_v, d)
    K2 = np.array(K, np.float64)
    V2 = np.array(V, np.float64)
    l_kv = np.asarray(l_kv, np.int64)
    l_next = l_kv.copy()
    for b in range(B):
        if l_kv[b] < l_max:
            K2[b, :, l_kv[b]] = k_new[b]
            V2[b, :, l_kv[b]] = v_new[b]
            l_next[b] = l_kv[b] + 1
    res = None
    if attention == "atopn":
        res = so.saga_decode_step(q, K2, V2, l_next, N, refresh_period, step, tau_in=tau_in, scale=scale)
        O = res.O
    elif attention == "dense":
        O = so.dense_gqa(q, K2, V2, l_next, scale=scale)
    else:
        raise ValueError("attention must be 'atopn' or 'dense'")
    y = linear(round_bf16(O.reshape(B, h_q * d)), w_o)
    return LayerResult(y, q, K2, V2, l_next, O, res)
