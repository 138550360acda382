"""Attention over the compressed history (fp64).

Sources: attention over a compressed cache of historical keys/values is the
repeated cost the method targets (NanoKV abstract); the NanoKV-Fast variant
scores queries directly on the stored coefficients instead of rebuilding full
keys ("mixed-dimensional attention", NanoKV project page, '03 / Measured
results').  Readings taken here:

* O = softmax(Q K^T * scale) V per head, no mask, every history key attended;
* the attention consumes the decoded cache rounded to the cache's storage
  dtype (bf16 caches are read as bf16(reconstruction), as a bf16 backbone
  attention would read them; fp32 caches as the fp32 reconstruction);
* mixed-dimensional scores for a key with centroid a and coefficients c:
  s = (q . C[a] + (B^T q) . c) * scale, which equals q . (C[a] + B c) * scale.

* with an uncompressed current chunk (the TempoKV page keeps the most recent frames
  uncompressed; quantized keys take attention mass from the unquantized current
  chunk): one softmax over the history keys followed by the chunk keys.

Pins (tests/test_oracle_attention.py): torch's fp64 scaled_dot_product_attention
on CPU, one key -> O = v, zero query -> mean of V, the mixed-dimensional identity
against scores computed from explicitly reconstructed keys, and for the chunk form
the log-sum-exp merge of the two parts' separate attentions.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_bf16


def cache_view(xhat_f32: np.ndarray, dtype: str) -> np.ndarray:
    """The decoded cache as attention reads it: bf16-rounded for bf16 caches."""
    if dtype == "bf16":
        return round_bf16(xhat_f32)
    return np.asarray(xhat_f32, dtype=np.float32)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, return_lse: bool = False):
    """Dense softmax attention in fp64.  q [Nq,H,d], k/v [Nk,H,d] -> O [Nq,H,d] (float64)."""
    q64, k64, v64 = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    nq, heads, _ = q64.shape
    out = np.empty((nq, heads, v64.shape[2]), dtype=np.float64)
    lse = np.empty((heads, nq), dtype=np.float64)
    for h in range(heads):
        s = (q64[:, h] @ k64[:, h].T) * scale
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        den = p.sum(axis=1, keepdims=True)
        out[:, h] = (p @ v64[:, h]) / den
        lse[h] = (m + np.log(den))[:, 0]
    return (out, lse) if return_lse else out


def attention_with_chunk(q: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray,
                         k_chunk: np.ndarray, v_chunk: np.ndarray, scale: float,
                         return_lse: bool = False):
    """Attention over the history keys/values followed by the current chunk's, fp64:
    the definition, one softmax over the concatenated keys."""
    return attention(q, np.concatenate([k_hist, k_chunk]), np.concatenate([v_hist, v_chunk]),
                     scale, return_lse)


def mixed_scores(q: np.ndarray, Ck: np.ndarray, idx: np.ndarray, B: np.ndarray,
                 chat: np.ndarray, scale: float) -> np.ndarray:
    """NanoKV-Fast style scores without rebuilding keys, fp64.

    q [Nq,H,d]; Ck [H,C,d]; idx [Nk,H]; B [d,m]; chat [Nk,H,m] -> [H,Nq,Nk]."""
    q64 = np.asarray(q, dtype=np.float64)
    C64 = np.asarray(Ck, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    c64 = np.asarray(chat, dtype=np.float64)
    nq, heads, _ = q64.shape
    out = np.empty((heads, nq, idx.shape[0]), dtype=np.float64)
    for h in range(heads):
        table = q64[:, h] @ C64[h].T          # q . C_j for every centroid
        proj = q64[:, h] @ B64                # B^T q
        out[h] = (table[:, idx[:, h]] + proj @ c64[:, h].T) * scale
    return out


def softmax_pv(scores: np.ndarray, v: np.ndarray, return_lse: bool = False):
    """softmax over keys of scores [H,Nq,Nk] (already scaled), times v [Nk,H,d] (fp64)."""
    v64 = np.asarray(v, dtype=np.float64)
    heads, nq, _ = scores.shape
    out = np.empty((nq, heads, v64.shape[2]), dtype=np.float64)
    lse = np.empty((heads, nq), dtype=np.float64)
    for h in range(heads):
        s = scores[h]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        den = p.sum(axis=1, keepdims=True)
        out[:, h] = (p @ v64[:, h]) / den
        lse[h] = (m + np.log(den))[:, 0]
    return (out, lse) if return_lse else out


def mixed_attention(q, Ck, idx, B, chat, v, scale, return_lse: bool = False):
    return softmax_pv(mixed_scores(q, Ck, idx, B, chat, scale), v, return_lse)
