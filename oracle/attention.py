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

* Jensen-bias correction (the INT2 Jensen-bias abstract on the Coral-KV listing page:
  quantization noise in the cached keys inflates their softmax weight through the
  convexity of exp; a per-score correction from the keys' quantization step sizes and
  the query, by a second-order Taylor expansion): a key quantized with step s_c on
  channel c carries noise e_c uniform on [-s_c/2, s_c/2] (variance s_c^2 / 12), so
  log E[exp(scale q . (k + e))] = scale q . k + (scale^2 / 2) sum_c q_c^2 s_c^2 / 12 to
  second order, and the corrected logit of a compressed key is
  scale q . k_hat - (scale^2 / 24) sum_g s_g^2 ||q_g||^2 over its scale groups g (one
  step per group).  Uncompressed current-chunk keys get no correction.  With the Hn
  rotation the noise is uniform in rotated coordinates; each rotation block lies inside
  one scale group and keeps the group's query norm, so the formula is unchanged.

Pins (tests/test_oracle_attention.py): torch's fp64 scaled_dot_product_attention
on CPU, one key -> O = v, zero query -> mean of V, the mixed-dimensional identity
against scores computed from explicitly reconstructed keys, for the chunk form
the log-sum-exp merge of the two parts' separate attentions, and for the Jensen
correction the exact log E[exp(a e)] = log(sinh(a s / 2) / (a s / 2)) of uniform
noise (agreement to fourth order), a Monte Carlo check that the corrected weights
are unbiased where the plain ones are not, and zero steps giving plain attention.
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


def jensen_correction(q: np.ndarray, step: np.ndarray, group: int, scale: float) -> np.ndarray:
    """(scale^2 / 24) sum_g s_g^2 ||q_g||^2 for every (head, query, key), fp64.

    q [Nq,H,d]; step [Nk,H,d/group] (the keys' group step sizes) -> [H,Nq,Nk]."""
    q64 = np.asarray(q, dtype=np.float64)
    s64 = np.asarray(step, dtype=np.float64)
    nq, heads, d = q64.shape
    qn = (q64.reshape(nq, heads, d // group, group) ** 2).sum(-1)      # [Nq,H,G] ||q_g||^2
    out = np.empty((heads, nq, s64.shape[0]), dtype=np.float64)
    for h in range(heads):
        out[h] = (scale * scale / 24.0) * (qn[:, h] @ (s64[:, h] ** 2).T)
    return out


def attention_jensen(q: np.ndarray, k: np.ndarray, v: np.ndarray, step: np.ndarray, group: int,
                     scale: float, k_chunk=None, v_chunk=None, return_lse: bool = False):
    """Softmax attention with the Jensen-bias correction subtracted from the logits of
    the compressed keys k (step sizes `step`), followed by the optional uncompressed
    chunk keys (no correction); fp64."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    heads = q64.shape[1]
    corr = jensen_correction(q64, step, group, scale)
    scores = np.stack([(q64[:, h] @ k64[:, h].T) * scale for h in range(heads)]) - corr
    vals = np.asarray(v, dtype=np.float64)
    if k_chunk is not None:
        kc = np.asarray(k_chunk, dtype=np.float64)
        sc = np.stack([(q64[:, h] @ kc[:, h].T) * scale for h in range(heads)])
        scores = np.concatenate([scores, sc], axis=2)
        vals = np.concatenate([vals, np.asarray(v_chunk, dtype=np.float64)])
    return softmax_pv(scores, vals, return_lse)
