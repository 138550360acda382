"""Low-dimensional residual coefficients (NanoKV / NanoKV-Fast key path).

Source: NanoKV abstract — shared content lives in cluster centres and joint
head-channel residuals are encoded into low-bit coefficients; NanoKV-Fast reuses
the stored coefficients for mixed-dimensional attention.  The pages give no
formula; readings taken here:

* a = nearest centroid (codec.assign), r = k - C[a] in fp32;
* coefficients c_j = sum_i B_ij * r_i, fp32, ascending i, multiply and add
  rounded separately, with the basis B [d][m] (orthonormal columns, stored in
  bf16) shared by all heads;
* c is quantized with the group quantizer at b bits and one group of m values
  per token-head;
* the reconstructed key is C[a] + B * dequant(c) (used only to check identities).

Pins (tests/test_oracle_coeff.py): with B = I (m = d) the coefficients equal the
plain residual bit for bit and the codec equals the centroid codec at group m;
coefficients of a residual lying in span(B) reconstruct it to quantization
error; fp64 matrix-product cross-check of the fixed-order sum.
"""
from __future__ import annotations

import numpy as np

from .codec import assign, quantize, dequantize, to_store


def coefficients(r: np.ndarray, B: np.ndarray) -> np.ndarray:
    """c = B^T r per token-head, fp32 ascending-order sum.  r [N,H,d], B [d,m] -> [N,H,m]."""
    r = np.asarray(r, dtype=np.float32)
    B = np.asarray(B, dtype=np.float32)
    acc = np.zeros(r.shape[:-1] + (B.shape[1],), dtype=np.float32)
    for i in range(r.shape[-1]):
        acc = acc + r[..., i:i + 1] * B[i]
    return acc


def encode_coeff(k: np.ndarray, Ck: np.ndarray, B: np.ndarray, bits: int) -> dict:
    """Centroid assignment + coefficient quantization (one group of m per token-head)."""
    k = np.asarray(k, dtype=np.float32)
    Ck = np.asarray(Ck, dtype=np.float32)
    idx, dist = assign(k, Ck)
    base = Ck[np.arange(Ck.shape[0])[None, :], idx]
    r = k - base
    c = coefficients(r, B)
    m = c.shape[-1]
    q, s16, z16 = quantize(c, bits, m)
    chat = dequantize(q, s16, z16, m)
    return dict(idx=idx, dist=dist, base=base, coeff=c, q=q, s16=s16, z16=z16, chat=chat,
                store=to_store(q, s16, z16, bits, idx, Ck.shape[1]))


def reconstruct_keys(Ck: np.ndarray, idx: np.ndarray, B: np.ndarray, chat: np.ndarray) -> np.ndarray:
    """K_hat = C[a] + B c_hat in fp64 (identity checks only).  -> [N,H,d]."""
    C64 = np.asarray(Ck, dtype=np.float64)
    base = C64[np.arange(C64.shape[0])[None, :], idx]
    return base + np.asarray(chat, dtype=np.float64) @ np.asarray(B, dtype=np.float64).T
