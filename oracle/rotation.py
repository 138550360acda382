"""Hn residual transform: an orthonormal Walsh-Hadamard rotation of each
non-overlapping group of n residual channels before the group quantizer.

Source: Coral-KV (arXiv 2610.12514) Fig. 5 (Hn transforms each non-overlapping
group of n residual channels independently; H16 / H64 compared at one shared
scale per 64 values) and Fig. 9b-c (H16 / H64 crossed with the scalar quantizer
at a fixed 64-value scale group).  The pages name the transform but print no
formula; the readings taken here are:

* H_n is the Sylvester Hadamard matrix (H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]),
  scaled by 1/sqrt(n) so that it is orthonormal and its own inverse;
* it acts on groups of n contiguous channels of one token-head residual vector
  (channels g*n .. g*n + n - 1 form group g);
* n is 16 or 64 (the two widths the pages compare); for these n, 1/sqrt(n) is a
  power of two, so the scaling is exact;
* the encoder rotates the fp32 residual r = x - base and quantizes the rotated
  vector; the decoder rotates the dequantized vector back (the same transform)
  and adds the base.

Arithmetic: the transform is evaluated by the Sylvester recursion itself, in
binary32: H_2m [a; b] = [H_m a + H_m b; H_m a - H_m b], each sum and difference
rounded once, the half-size products evaluated first, then the 1/sqrt(n) scale.
Its rounded result therefore depends only on this recursion, which also fixes the
order in which a faster butterfly network has to combine the values to reproduce
it exactly (pairs at distance 1 first, then 2, 4, ..., n/2).

Pins (tests/test_oracle_rotation.py): exact agreement with the integer matrix
product H_n x for small-integer inputs (against scipy.linalg.hadamard and against
the entries (-1)^popcount(i & j) built independently), the fp64 matrix product within
the binary32 rounding bound on random inputs, self-inverse, norm preservation,
block-diagonal action on a 128-channel vector, exact round trip of encode/decode for
residuals that sit on the quantization grid after the rotation (where the unrotated
codec is not exact), the reconstruction error bound of the rotated codec, and the
rotated-coordinate form of attention (queries and centroid tables rotated, output
rotated back) against attention over the decoded cache.
"""
from __future__ import annotations

import numpy as np

WIDTHS = (16, 64)


def _sylvester_apply(a: np.ndarray) -> np.ndarray:
    """Unnormalized H_m a over the last axis (m a power of two), binary32,
    by the Sylvester recursion."""
    m = a.shape[-1]
    if m == 1:
        return a
    lo = _sylvester_apply(a[..., : m // 2])
    hi = _sylvester_apply(a[..., m // 2:])
    return np.concatenate([lo + hi, lo - hi], axis=-1)


def rotate(x: np.ndarray, n: int) -> np.ndarray:
    """(H_n / sqrt(n)) applied to every group of n contiguous channels of the last
    axis.  x: [..., d] float32 with n dividing d -> float32 [..., d]."""
    if n not in WIDTHS:
        raise ValueError("rotation width must be 16 or 64")
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    if d % n:
        raise ValueError("rotation width must divide the vector length")
    g = x.reshape(*x.shape[:-1], d // n, n)
    y = _sylvester_apply(g) * np.float32(1.0 / np.sqrt(n))
    return y.reshape(x.shape).astype(np.float32)
