"""Linear predictors that form the codec's base from reconstructed state.

Sources:
* Coral-KV (arXiv 2610.12514) Fig. 3: at layer l > 0 the reconstructed layer
  l-1 feeds the predictors; keys are predicted from K_{l-1}, values from
  [K_l, V_{l-1}]; both maps are a per-head block-diagonal part plus a global
  rank-r part (block-DPLR); the quantized residual is added to the prediction.
  Layer 0 is an INT4 anchor (Coral-KV Fig. 8).
* TempoKV (arXiv 2610.15324) Fig. 2b: K_{t,s} is predicted from the
  reconstructed key history, V_{t,s} from the aligned reconstructed key plus
  the reconstructed value history; only the low-bit residual is stored.  The
  anchor frame uses 4 bits (TempoKV Table 7).

Readings taken here (the pages give no formulas):
* predictor inputs are the reconstructions rounded to bf16 (the decoded cache
  in its storage dtype);
* block-DPLR: pred[h] = W_h xin_h + (U (Vlr^T xlr))[h], where xin_h stacks the
  head's channels of every input and xlr stacks every input over all heads;
  evaluated exactly (fp64) and rounded once to fp32 to become the base;
* temporal keys: pred = (a * K_{t-1}) + (b * K_{t-2}) per channel in fp32
  (three rounded operations), with K_{-1} := K_0 at t = 1;
* temporal values: pred = M_h K_t + beta * V_{t-1}, exact (fp64), rounded once
  to fp32, with V_{-1} := 0.

Pins (tests/test_oracle_predict.py): W = I, U = 0 reduces the DPLR predictor to
previous-layer DPCM; a = 1, b = 0 reduces the temporal key predictor to
previous-frame DPCM; M = 0 reduces the value predictor to a scaled previous
frame; the block-DPLR map equals the dense (H*d)x(n*H*d) matrix assembled from
its blocks and factors and a per-element brute force; the temporal value map equals
a per-element sum in exact rational arithmetic with a non-symmetric M_h (a transposed
M_h fails); the temporal chain's first predicted frame reads the anchor's
reconstruction for both key terms (b != 0, so K_{-1} = 0 fails); chains reproduce
their inputs within the O(s/2) quantization bound; with an Hn rotation of the
prediction residuals, inputs whose rotated residual sits on the quantization grid are
reconstructed exactly (and not without the rotation), and the reconstruction error
keeps the rotated quantizer's bound.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_bf16
from .codec import quantize, dequantize, to_store
from .rotation import rotate


def dplr_predict(inputs, W: np.ndarray, U: np.ndarray, Vlr: np.ndarray) -> np.ndarray:
    """Block-DPLR prediction, exact in fp64.

    inputs: list of reconstructions [N,H,d] float32 (rounded to bf16 here);
    W [H, d, n_in*d]; U [H*d, r]; Vlr [n_in*H*d, r]  ->  [N,H,d] float64."""
    xs = [round_bf16(x).astype(np.float64) for x in inputs]
    n, heads, d = xs[0].shape
    xin = np.concatenate(xs, axis=2)                          # [N, H, n_in*d]
    W64 = np.asarray(W, dtype=np.float64)
    block = np.stack([xin[:, h] @ W64[h].T for h in range(heads)], axis=1)
    xlr = np.concatenate([x.reshape(n, heads * d) for x in xs], axis=1)
    t = xlr @ np.asarray(Vlr, dtype=np.float64)               # rank-r intermediate, exact
    low = (t @ np.asarray(U, dtype=np.float64).T).reshape(n, heads, d)
    return block + low


def dplr_dense_matrix(W: np.ndarray, U: np.ndarray, Vlr: np.ndarray, n_in: int) -> np.ndarray:
    """The full (H*d) x (n_in*H*d) matrix of the block-DPLR map (pin helper)."""
    heads, d, _ = W.shape
    D = heads * d
    M = np.asarray(U, dtype=np.float64) @ np.asarray(Vlr, dtype=np.float64).T
    for h in range(heads):
        for j in range(n_in):
            M[h * d:(h + 1) * d, j * D + h * d:j * D + (h + 1) * d] += \
                np.asarray(W[h][:, j * d:(j + 1) * d], dtype=np.float64)
    return M


def temporal_predict_k(k1: np.ndarray, k2: np.ndarray, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """(a * bf16(K_{t-1})) + (b * bf16(K_{t-2})) in fp32.  a, b: [H, d] float32."""
    x1 = round_bf16(k1)
    x2 = round_bf16(k2)
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    return (a * x1) + (b * x2)


def temporal_predict_v(k_t: np.ndarray, v1: np.ndarray, M: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """M_h bf16(K_t) + beta * bf16(V_{t-1}), exact (fp64).  M [H,d,d], beta [H,d]."""
    x = round_bf16(k_t).astype(np.float64)
    y = round_bf16(v1).astype(np.float64)
    M64 = np.asarray(M, dtype=np.float64)
    cross = np.stack([x[:, h] @ M64[h].T for h in range(x.shape[1])], axis=1)
    return cross + np.asarray(beta, dtype=np.float64) * y


def encode_with_prediction(x: np.ndarray, pred: np.ndarray, bits: int, group: int,
                           rotation: int = 0) -> dict:
    """Base = fp32(prediction); residual, quantize, reconstruct (fp32).  With
    `rotation` = n the prediction residual is rotated by H_n / sqrt(n) per group of n
    channels before it is quantized, and the dequantized vector rotated back before the
    base is added (Coral-KV Fig. 5 and Fig. 9b-c: Hn applied to the prediction
    residuals)."""
    base = np.asarray(pred, dtype=np.float64).astype(np.float32)
    r = np.asarray(x, dtype=np.float32) - base
    if rotation:
        r = rotate(r, rotation)
    q, s16, z16 = quantize(r, bits, group)
    deq = dequantize(q, s16, z16, group)
    if rotation:
        deq = rotate(deq, rotation)
    xhat = base + deq
    return dict(base=base, q=q, s16=s16, z16=z16, xhat=xhat, store=to_store(q, s16, z16, bits))


def dplr_chain(layers, params: dict, bits: int, group: int, anchor_bits: int,
               anchor_group: int | None = None, teacher=None, rotation: int = 0):
    """Cross-layer chain over `layers` = iterable of (K_l, V_l) float32 [N,H,d].

    Layer 0 is the anchor (base 0, `anchor_bits`).  Layer l >= 1 predicts K_l from
    K_hat_{l-1} and V_l from [K_hat_l, V_hat_{l-1}].  With `teacher` (an iterable of
    (K_hat_{l}, V_hat_{l}) reconstructions), predictions read the teacher's state
    instead of the chain's own.  `rotation` (16 or 64) rotates the prediction residuals
    of layers l >= 1 (the anchor is not rotated).  Yields one dict per layer."""
    anchor_group = anchor_group or group
    kprev = vprev = None
    tit = iter(teacher) if teacher is not None else None
    for layer, (k, v) in enumerate(layers):
        if layer == 0:
            zero = np.zeros_like(np.asarray(k, dtype=np.float32))
            ek = encode_with_prediction(k, zero, anchor_bits, anchor_group)
            ev = encode_with_prediction(v, zero, anchor_bits, anchor_group)
        else:
            kp = dplr_predict([kprev], params["WK"], params["UK"], params["VK"])
            ek = encode_with_prediction(k, kp, bits, group, rotation)
            vp = dplr_predict([ek["xhat"], vprev], params["WV"], params["UV"], params["VV"])
            ev = encode_with_prediction(v, vp, bits, group, rotation)
        yield dict(layer=layer, k=ek, v=ev)
        if tit is not None:
            kprev, vprev = next(tit)
        else:
            kprev, vprev = ek["xhat"], ev["xhat"]


def temporal_chain(k_frames, v_frames, a, b, M, beta, bits: int, group: int, anchor_bits: int,
                   anchor_group: int | None = None, rotation: int = 0):
    """TempoKV-style chain over frames (lists of [T,H,d] float32).  Frame 0 is the anchor.
    `rotation` (16 or 64) rotates the prediction residuals of frames t >= 1.  Yields
    per-frame dicts with the key and value encodings."""
    anchor_group = anchor_group or group
    k1 = k2 = v1 = None
    for t, (k, v) in enumerate(zip(k_frames, v_frames)):
        if t == 0:
            zero = np.zeros_like(np.asarray(k, dtype=np.float32))
            ek = encode_with_prediction(k, zero, anchor_bits, anchor_group)
            ev = encode_with_prediction(v, zero, anchor_bits, anchor_group)
        else:
            kp = temporal_predict_k(k1, k2 if t > 1 else k1, a, b)
            ek = encode_with_prediction(k, kp, bits, group, rotation)
            vp = temporal_predict_v(ek["xhat"], v1, M, beta)
            ev = encode_with_prediction(v, vp, bits, group, rotation)
        yield dict(frame=t, k=ek, v=ev)
        k2, k1, v1 = k1, ek["xhat"], ev["xhat"]
