"""Residual codec: nearest-centroid base, group-wise INTb quantizer, packing, decode.

Sources: clustering-based KV quantization groups similar key/value vectors and
quantizes the residual errors (Coral-KV abstract; NanoKV abstract, "shared
content in cluster centers"); centroids per cache block (Coral-KV Fig. 2c); a
shared scale per group of values (Coral-KV Fig. 5c, "one shared scale per 64
values"); the stored state is residual codes + scales + assignments + codebooks
(Coral-KV Table 9 caption).  The pages fix none of the arithmetic; the readings
taken here are:

* distance: d_j = sum_i (x_i - c_ji)^2, fp32, ascending i, each of the
  subtract / square / accumulate steps rounded separately;
* argmin ties go to the lowest centroid index;
* per group of ``g`` contiguous channels of one token-head vector:
  z = fp16(min), s = fp16(fp32(max - min) / (2^b - 1)),
  q = clamp(rint((r - z) / s), 0, 2^b - 1) (q = 0 when s == 0),
  dequant = (q * s) + z, reconstruction = base + dequant;
* packing: element i -> word floor(i*b/32), bit offset b*(i mod 32/b)
  (little-endian); scale/zero word = fp16 bits of s | fp16 bits of z << 16;
  index stored as uint8 when there are at most 256 centroids, else uint16;
* store layout is head-major: codes [H][N][d*b/32], scale_zero [H][N][d/g],
  index [H][N].

Pins (tests/test_oracle_codec.py): brute-force fp64 argmin on tiny inputs,
one-centroid and duplicate-centroid cases, the s/2 round-trip bound on groups
built on an fp16 grid, exact reconstruction of grid values, exact zero residual
when the input equals its base, exhaustive pack/unpack over every code and
position, and hand-written packed words in tests/golden/.
"""
from __future__ import annotations

import numpy as np

from .numerics import f16
from .rotation import rotate


# ------------------------------- assignment -------------------------------

def sq_dist(x: np.ndarray, C: np.ndarray, token_chunk: int = 128) -> np.ndarray:
    """Squared distances, fp32, ascending channel order.

    For every (token, head, centroid): acc = 0; for i = 0..d-1:
    t = x_i - c_i; acc = acc + t*t (each operation rounded to fp32).
    Tokens are processed in chunks only to keep the temporaries in cache.

    x: [N, H, d] float32, C: [H, K, d] float32 -> [N, H, K] float32."""
    x = np.asarray(x, dtype=np.float32)
    C = np.asarray(C, dtype=np.float32)
    n, h, d = x.shape
    k = C.shape[1]
    xt = np.ascontiguousarray(np.transpose(x, (2, 0, 1)))   # [d, N, H]
    ct = np.ascontiguousarray(np.transpose(C, (2, 0, 1)))   # [d, H, K]
    out = np.empty((n, h, k), dtype=np.float32)
    for s in range(0, n, token_chunk):
        e = min(n, s + token_chunk)
        acc = np.zeros((e - s, h, k), dtype=np.float32)
        t = np.empty_like(acc)
        for i in range(d):
            np.subtract(xt[i, s:e, :, None], ct[i][None], out=t)
            np.multiply(t, t, out=t)
            np.add(acc, t, out=acc)
        out[s:e] = acc
    return out


def assign(x: np.ndarray, C: np.ndarray):
    """Nearest centroid per (token, head); ties -> lowest index.  Returns (idx [N,H], dist)."""
    dist = sq_dist(x, C)
    return np.argmin(dist, axis=-1), dist  # argmin returns the first minimum


def tie_gap(dist: np.ndarray) -> np.ndarray:
    """Relative gap (d2 - d1) / d1 between the two smallest distances (fp64).

    +inf when there is a single centroid, or d1 == 0 < d2; 0 when d1 == d2 == 0."""
    if dist.shape[-1] < 2:
        return np.full(dist.shape[:-1], np.inf)
    part = np.sort(dist.astype(np.float64), axis=-1)
    d1, d2 = part[..., 0], part[..., 1]
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = (d2 - d1) / d1
    gap = np.where(d1 > 0, gap, np.where(d2 > 0, np.inf, 0.0))
    return gap


# ------------------------------- quantizer -------------------------------

def quantize(r: np.ndarray, bits: int, group: int):
    """Group-wise asymmetric INTb quantizer on the last axis.

    r: [..., d] float32 -> (q uint8 [..., d], s16 float16 [..., d/g], z16 float16 [..., d/g])."""
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    r = np.asarray(r, dtype=np.float32)
    d = r.shape[-1]
    if d % group:
        raise ValueError("group must divide the vector length")
    levels = np.float32((1 << bits) - 1)
    rg = r.reshape(*r.shape[:-1], d // group, group)
    mn = rg.min(axis=-1)
    mx = rg.max(axis=-1)
    z16 = f16(mn)
    with np.errstate(over="ignore"):
        s32 = (mx - mn) / levels
        s16 = f16(s32)
    if not (np.all(np.isfinite(s16)) and np.all(np.isfinite(z16))):
        raise OverflowError("group range exceeds the fp16 scale/zero format")
    z = z16.astype(np.float32)[..., None]
    s = s16.astype(np.float32)[..., None]
    num = rg - z
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.rint(num / s)
    qf = np.where(s == 0, np.float32(0), np.clip(qf, np.float32(0), levels))
    return qf.astype(np.uint8).reshape(r.shape), s16, z16


def dequantize(q: np.ndarray, s16: np.ndarray, z16: np.ndarray, group: int) -> np.ndarray:
    """(q * s) + z in fp32, two rounded operations.  Returns float32 [..., d]."""
    d = q.shape[-1]
    qf = q.astype(np.float32).reshape(*q.shape[:-1], d // group, group)
    s = np.asarray(s16, dtype=np.float16).astype(np.float32)[..., None]
    z = np.asarray(z16, dtype=np.float16).astype(np.float32)[..., None]
    prod = qf * s
    return (prod + z).reshape(q.shape)


# ------------------------------- packing -------------------------------

def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """[..., d] codes -> [..., d*bits/32] uint32, element i at word i*bits//32, bit bits*(i%per)."""
    per = 32 // bits
    d = q.shape[-1]
    if (d * bits) % 32:
        raise ValueError("d*bits must be a multiple of 32")
    qq = np.asarray(q).astype(np.uint32).reshape(*q.shape[:-1], d // per, per)
    shifts = (np.uint32(bits) * np.arange(per, dtype=np.uint32))
    return np.bitwise_or.reduce(qq << shifts, axis=-1).astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of pack_codes."""
    per = 32 // bits
    shifts = (np.uint32(bits) * np.arange(per, dtype=np.uint32))
    w = np.asarray(words, dtype=np.uint32)
    q = (w[..., :, None] >> shifts) & np.uint32((1 << bits) - 1)
    return q.reshape(*w.shape[:-1], d).astype(np.uint8)


def pack_scale_zero(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    s = np.asarray(s16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(z16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return s | (z << np.uint32(16))


def unpack_scale_zero(w: np.ndarray):
    w = np.asarray(w, dtype=np.uint32)
    s16 = (w & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z16 = (w >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return s16, z16


def index_dtype(n_centroids: int):
    return np.uint8 if n_centroids <= 256 else np.uint16


# ------------------------------- encode / decode -------------------------------

def to_store(q, s16, z16, bits: int, idx=None, n_centroids: int | None = None) -> dict:
    """Natural [N][H][...] codec outputs -> head-major packed store."""
    codes = np.ascontiguousarray(np.transpose(pack_codes(q, bits), (1, 0, 2)))
    sz = np.ascontiguousarray(np.transpose(pack_scale_zero(s16, z16), (1, 0, 2)))
    out = dict(codes=codes, scale_zero=sz, index=None)
    if idx is not None:
        out["index"] = np.ascontiguousarray(idx.T.astype(index_dtype(n_centroids)))
    return out


def encode_residual(x: np.ndarray, base: np.ndarray, bits: int, group: int,
                    rotation: int = 0) -> dict:
    """r = x - base (fp32), optionally rotated by H_n / sqrt(n) per group of n
    channels (n = ``rotation``, see rotation.py), quantize.  x, base: [N, H, d] float32."""
    r = np.asarray(x, dtype=np.float32) - np.asarray(base, dtype=np.float32)
    if rotation:
        r = rotate(r, rotation)
    q, s16, z16 = quantize(r, bits, group)
    return dict(q=q, s16=s16, z16=z16, base=np.asarray(base, dtype=np.float32))


def encode_centroid(x: np.ndarray, C: np.ndarray, bits: int, group: int,
                    rotation: int = 0) -> dict:
    """Centroid base: a = argmin ||x - C_a||^2, base = C[a] (the assignment is made on
    the unrotated vectors).  Returns natural-layout outputs plus the packed head-major
    ``store``."""
    x = np.asarray(x, dtype=np.float32)
    C = np.asarray(C, dtype=np.float32)
    idx, dist = assign(x, C)
    base = C[np.arange(C.shape[0])[None, :], idx]
    out = encode_residual(x, base, bits, group, rotation)
    out.update(idx=idx, dist=dist)
    out["store"] = to_store(out["q"], out["s16"], out["z16"], bits, idx, C.shape[1])
    return out


def encode_none(x: np.ndarray, bits: int, group: int) -> dict:
    """Anchor / plain group quantization: base = 0."""
    x = np.asarray(x, dtype=np.float32)
    out = encode_residual(x, np.zeros_like(x), bits, group)
    out["store"] = to_store(out["q"], out["s16"], out["z16"], bits)
    return out


def decode_store(store: dict, bits: int, group: int, d: int, base: np.ndarray | None = None,
                 C: np.ndarray | None = None, rotation: int = 0) -> np.ndarray:
    """Reconstruction base + ((q * s) + z) from a head-major store, as [N][H][d] float32;
    with ``rotation`` = n the dequantized vector is rotated back by H_n / sqrt(n) (its
    own inverse) before the base is added.

    The base is given explicitly, or gathered from centroids C [H][K][d] via the index."""
    q = np.transpose(unpack_codes(store["codes"], bits, d), (1, 0, 2))
    s16, z16 = unpack_scale_zero(np.transpose(store["scale_zero"], (1, 0, 2)))
    deq = dequantize(q, s16, z16, group)
    if rotation:
        deq = rotate(deq, rotation)
    if base is None:
        if C is None:
            base = np.zeros_like(deq)
        else:
            idx = store["index"].T.astype(np.int64)
            base = np.asarray(C, dtype=np.float32)[np.arange(C.shape[0])[None, :], idx]
    return np.asarray(base, dtype=np.float32) + deq
