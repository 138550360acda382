"""Online centroid fitting at block fill: Lloyd iterations on the tokens of one cache
block, per head.

Source: Coral-KV (arXiv 2610.12514) Fig. 2c — QVG fits video-specific centroids online
when a cache block reaches its token limit (the clustering-based baseline whose
centroids the codec's nearest-centroid base uses); the NanoKV abstract's cluster
centers.  The pages name the step, not its algorithm; the readings taken here:

* the fit is k-means by Lloyd's iterations, started from centroids the caller gives
  (for instance tokens of the block at a stride) and run a fixed number of times;
* the assignment step is the codec's own nearest-centroid search (fp32 squared
  distance, ascending channels, ties to the lowest index), so the fitted table is
  the one the encoder will search;
* the update step sets every centroid that received tokens to the mean of its
  tokens, and rounds it to the table's storage type (bf16 here, nearest even); a
  centroid that received none keeps its value;
* the mean is the exact one (fp64 sum over the tokens, divided by their count), then
  rounded to fp32 and to bf16.

Pins (tests/test_oracle_fit.py): well-separated blobs reach their rounded means in one
step from one seed per blob; a duplicate centroid stays empty and unchanged (ties go to
the lower index); one centroid becomes the rounded global mean; every step's output
satisfies its own definition (each non-empty centroid is the rounded mean of the tokens
the codec search assigns to it); the k-means objective does not grow by more than the
bf16 rounding of the centroids from one iteration to the next; a worked example fixes
the rounding of the mean (exact mean 1 + 2^-8 + 2^-30 becomes fp32 1 + 2^-8, a bf16
tie, so 1 - not the 1 + 2^-7 that a single rounding gives).
"""
from __future__ import annotations

import numpy as np

from .codec import assign
from .numerics import round_bf16


def lloyd_step(x: np.ndarray, C: np.ndarray):
    """One iteration.  x [N,H,d] float32 (bf16 values), C [H,K,d] float32 (bf16 values)
    -> (new C [H,K,d] float32 holding bf16 values, assignments [N,H], counts [H,K])."""
    x = np.asarray(x, dtype=np.float32)
    C = np.asarray(C, dtype=np.float32)
    idx, _ = assign(x, C)
    heads, k, d = C.shape
    new = C.copy()
    counts = np.zeros((heads, k), dtype=np.int64)
    for h in range(heads):
        for j in range(k):
            members = x[idx[:, h] == j, h].astype(np.float64)
            counts[h, j] = members.shape[0]
            if members.shape[0]:
                mean = members.sum(axis=0) / members.shape[0]
                new[h, j] = round_bf16(mean.astype(np.float32))
    return new, idx, counts


def fit(x: np.ndarray, C0: np.ndarray, iterations: int):
    """`iterations` Lloyd steps from C0; returns the fitted table (float32 bf16 values)."""
    C = np.asarray(C0, dtype=np.float32)
    for _ in range(iterations):
        C, _, _ = lloyd_step(x, C)
    return C


def objective(x: np.ndarray, C: np.ndarray) -> float:
    """Sum over tokens and heads of the squared distance to the nearest centroid (fp64)."""
    x64 = np.asarray(x, dtype=np.float64)
    C64 = np.asarray(C, dtype=np.float64)
    total = 0.0
    for h in range(C64.shape[0]):
        dist = ((x64[:, h, None, :] - C64[h][None]) ** 2).sum(-1)
        total += float(dist.min(axis=1).sum())
    return total
