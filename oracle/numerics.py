"""Storage-type conversions for the oracle (numpy only).

bf16 rounding is written out with uint32 bit operations (round to nearest,
ties to even); fp16 rounding uses numpy's float32 -> float16 cast, which is
round-to-nearest-even with subnormals.  Pinned in the tests against torch's
own bfloat16 cast and against hand-built tie cases.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def round_bf16(x) -> np.ndarray:
    """float32 value rounded to the nearest bf16, returned as float32."""
    return bf16_to_f32(f32_to_bf16(x))


def f16(x) -> np.ndarray:
    """float32 -> float16, round to nearest even (numpy's cast); overflow gives inf."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def as_f32(x, dtype: str) -> np.ndarray:
    """Input tensor in its storage form ('f32' array or 'bf16' uint16 bits) as float32."""
    if dtype == "bf16":
        return bf16_to_f32(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")
