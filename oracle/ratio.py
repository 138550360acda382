"""Closed-form storage cost of the compressed cache.

Bits per element = b (residual code) + 32/g (fp16 scale + fp16 zero per group)
+ index bits / d (centroid assignment per token-head) + shared parameters
(centroids, predictors, basis) / (tokens * d) + anchor fraction * (anchor
cost - residual cost).  Compression ratio = source bits / bits per element
(16 for bf16 caches, 32 for fp32).

Pinned by figures the pages print (tests/golden/compression_ratios.json):
the INT2 and INT4 per-group baselines of the TempoKV tables (5.33x, 3.20x),
NanoKV's nominal 32x coefficient compression, and the linear dependence of
TempoKV's compression on anchor bits (TempoKV appendix Table 7).
"""
from __future__ import annotations

import math


def residual_bits(bits: int, group: int, sz_bits: int = 32) -> float:
    """Code bits plus the per-group scale/zero overhead, per element."""
    return bits + sz_bits / group


def bits_per_element(bits: int, group: int, dim: int, *, index_bits: float = 0.0,
                     shared_bits: float = 0.0, n_tokens: int | None = None,
                     anchor_fraction: float = 0.0, anchor_bits: int | None = None,
                     anchor_group: int | None = None) -> float:
    per = residual_bits(bits, group)
    if anchor_fraction:
        anchor = residual_bits(anchor_bits, anchor_group or group)
        per = (1.0 - anchor_fraction) * per + anchor_fraction * anchor
    per += index_bits / dim
    if shared_bits:
        per += shared_bits / (n_tokens * dim)
    return per


def coeff_bits_per_element(coeff_dim: int, bits: int, dim: int, group: int | None = None,
                           sz: bool = True) -> float:
    """Key coefficient storage per original element: m*b/d (+ scale/zero per group of m)."""
    group = group or coeff_dim
    per = coeff_dim * bits / dim
    if sz:
        per += (coeff_dim / group) * 32 / dim
    return per


def information_index_bits(n_centroids: int) -> int:
    return max(0, math.ceil(math.log2(n_centroids)))


def stored_index_bits(n_centroids: int) -> int:
    return 8 if n_centroids <= 256 else 16


def ratio(bits_per_elem: float, source_bits: int = 16) -> float:
    return source_bits / bits_per_elem
