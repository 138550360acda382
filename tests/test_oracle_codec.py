"""Pins for the codec oracle: brute force, closed forms, special cases and the
hand-worked examples in tests/golden/codec_small.json."""
import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import codec


def _golden():
    with open(os.path.join(GOLDEN, "codec_small.json")) as f:
        return json.load(f)


# ------------------------------ assignment ------------------------------

def test_assignment_golden_examples():
    g = _golden()["assignment"]
    C = np.array(g["centroids"], dtype=np.float32)[None]          # one head
    x = np.array(g["points"], dtype=np.float32)[:, None, :]
    idx, _ = codec.assign(x, C)
    assert idx[:, 0].tolist() == g["index"]


@pytest.mark.parametrize("seed", range(5))
def test_assignment_matches_fp64_brute_force(seed):
    rng = np.random.default_rng(seed)
    n, h, k, d = 300, 3, 24, 16
    x = (rng.standard_normal((n, h, d)) * 3).astype(np.float32)
    C = (rng.standard_normal((h, k, d)) * 3).astype(np.float32)
    idx, dist = codec.assign(x, C)
    # fp64 brute force written independently: norm of the difference vector
    for t in range(n):
        for hh in range(h):
            d64 = np.array([np.linalg.norm(x[t, hh].astype(np.float64) - C[hh, j]) ** 2
                            for j in range(k)])
            best = int(np.argmin(d64))
            if idx[t, hh] != best:
                # only a near tie may differ, and then by less than the fp32 rounding
                assert abs(d64[idx[t, hh]] - d64[best]) <= 1e-5 * d64[best]
            assert abs(dist[t, hh, best] - d64[best]) <= 1e-5 * max(d64[best], 1e-30)


def test_assignment_one_centroid_and_duplicates():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 2, 8)).astype(np.float32)
    C1 = rng.standard_normal((2, 1, 8)).astype(np.float32)
    idx, dist = codec.assign(x, C1)
    assert np.all(idx == 0)
    assert np.all(np.isinf(codec.tie_gap(dist)))
    # duplicates: centroid 5 is a copy of centroid 2; ties go to the lower index
    C = rng.standard_normal((2, 8, 8)).astype(np.float32)
    C[:, 5] = C[:, 2]
    x2 = C[:, 2][None] + np.float32(1e-3)
    idx2, dist2 = codec.assign(np.repeat(x2, 4, axis=0), C)
    assert np.all(idx2 == 2)
    assert np.all(codec.tie_gap(dist2) == 0.0)


def test_tie_gap_special_cases():
    dist = np.array([[[0.0, 0.0, 1.0]], [[0.0, 2.0, 3.0]], [[2.0, 3.0, 2.0]]], dtype=np.float32)
    gap = codec.tie_gap(dist)
    assert gap[0, 0] == 0.0 and np.isinf(gap[1, 0]) and gap[2, 0] == 0.0
    dist = np.array([[[4.0, 5.0]]], dtype=np.float32)
    assert codec.tie_gap(dist)[0, 0] == pytest.approx(0.25)


def test_distance_is_ascending_fp32_sum():
    # a case where summation order changes the fp32 result: 1e8 then many 1's
    x = np.zeros((1, 1, 5), dtype=np.float32)
    C = np.array([[[1e4, 1.0, 1.0, 1.0, 1.0]]], dtype=np.float32)
    d = codec.sq_dist(x, C)[0, 0, 0]
    acc = np.float32(0)
    for v in (1e8, 1.0, 1.0, 1.0, 1.0):
        acc = np.float32(acc + np.float32(v))
    assert d == acc == np.float32(1e8)   # each +1 is absorbed in ascending order


# ------------------------------ quantizer ------------------------------

@pytest.mark.parametrize("ex", _golden()["examples"], ids=lambda e: e["name"])
def test_golden_codec_examples(ex):
    r = np.array(ex["residual"], dtype=np.float32)[None]
    q, s16, z16 = codec.quantize(r, ex["bits"], ex["group"])
    assert q[0].tolist() == ex["codes"]
    words = codec.pack_codes(q, ex["bits"])
    assert [f"0x{w:08X}" for w in words[0]] == ex["words"]
    sz = codec.pack_scale_zero(s16, z16)
    assert [f"0x{w:08X}" for w in sz[0]] == ex["scale_zero"]
    deq = codec.dequantize(q, s16, z16, ex["group"])
    assert deq[0].tolist() == [float(v) for v in ex["decoded"]]


@pytest.mark.parametrize("bits", [2, 4])
def test_grid_values_reconstruct_exactly(bits):
    """x = z + k*s with s, z exact fp16 and k covering 0 and L: codes == k, exact decode."""
    rng = np.random.default_rng(bits)
    L = (1 << bits) - 1
    n, g = 400, 32
    s = codec.f16(rng.uniform(0.01, 2.0, n)).astype(np.float32)
    z = codec.f16(rng.uniform(-5, 5, n)).astype(np.float32)
    k = rng.integers(0, L + 1, (n, g))
    k[:, 0], k[:, 1] = 0, L
    x = (z[:, None] + k * s[:, None].astype(np.float64)).astype(np.float32)
    exact = np.array_equal(x.astype(np.float64), z[:, None] + k * s[:, None].astype(np.float64))
    assert exact  # the grid points are representable
    q, s16, z16 = codec.quantize(x, bits, g)
    assert np.array_equal(q, k.astype(np.uint8))
    assert np.array_equal(codec.dequantize(q, s16, z16, g), x)


@pytest.mark.parametrize("bits,group", [(2, 32), (4, 32), (2, 64), (4, 16)])
def test_round_trip_half_scale_bound_on_fp16_grid_ends(bits, group):
    """When min, max and the scale are exact in fp16, |r - r_hat| <= s/2 (+ fp32 rounding)."""
    rng = np.random.default_rng(10 + bits + group)
    L = (1 << bits) - 1
    n = 500
    s = codec.f16(rng.uniform(0.01, 1.0, n)).astype(np.float32)
    z = codec.f16(rng.uniform(-3, 3, n)).astype(np.float32)
    hi = (z.astype(np.float64) + L * s.astype(np.float64)).astype(np.float32)
    inner = rng.uniform(0, 1, (n, group)) * (hi - z)[:, None] + z[:, None]
    x = inner.astype(np.float32)
    x[:, 0], x[:, -1] = z, hi
    q, s16, z16 = codec.quantize(x, bits, group)
    assert np.array_equal(s16.astype(np.float32)[:, 0], s) and np.array_equal(z16.astype(np.float32)[:, 0], z)
    err = np.abs(codec.dequantize(q, s16, z16, group).astype(np.float64) - x)
    tol = s[:, None] / 2 + 4 * np.spacing(np.maximum(np.abs(x), np.abs(hi)[:, None]).astype(np.float32))
    assert np.all(err <= tol)


@pytest.mark.parametrize("bits,group", [(2, 32), (4, 32), (2, 64), (4, 64)])
def test_round_trip_general_bound(bits, group):
    """Random data: |r - r_hat| <= max(s/2, z - min, L*(s32 - s16) + (min - z)) + rounding,
    the bound that accounts for fp16 rounding of the scale and zero."""
    rng = np.random.default_rng(20 + bits)
    L = (1 << bits) - 1
    x = (rng.standard_normal((2000, group)) * rng.uniform(0.01, 50, (2000, 1))).astype(np.float32)
    q, s16, z16 = codec.quantize(x, bits, group)
    mn, mx = x.min(1).astype(np.float64), x.max(1).astype(np.float64)
    s, z = s16[:, 0].astype(np.float64), z16[:, 0].astype(np.float64)
    s32 = (mx - mn) / L
    bound = np.maximum.reduce([s / 2, z - mn, L * (s32 - s) + (mn - z)])
    err = np.abs(codec.dequantize(q, s16, z16, group).astype(np.float64) - x).max(1)
    slack = 8 * np.spacing(np.abs(x).max(1).astype(np.float32)).astype(np.float64)
    assert np.all(err <= bound + slack)
    # the s/2 bound is what holds almost everywhere
    frac_over = np.mean(np.abs(codec.dequantize(q, s16, z16, group) - x) > (s16.astype(np.float32) / 2 + 1e-6 * np.abs(x).max()))
    assert frac_over < 0.01


def test_zero_residual_is_exact():
    rng = np.random.default_rng(5)
    base = rng.standard_normal((64, 3, 128)).astype(np.float32)
    out = codec.encode_residual(base, base, 2, 32)
    assert np.all(out["q"] == 0)
    assert np.all(out["s16"] == 0) and np.all(out["z16"] == 0)
    assert np.array_equal(codec.decode_store(codec.to_store(out["q"], out["s16"], out["z16"], 2),
                                             2, 32, 128, base=base), base)


def test_clamp_when_zero_rounds_above_min():
    # min = 1 + 3*2^-12 rounds up to fp16 1 + 2^-10; that element must clamp to code 0
    mn = np.float32(1 + 3 * 2.0 ** -12)
    r = np.full((1, 16), 2.0, dtype=np.float32)
    r[0, 0] = mn
    q, s16, z16 = codec.quantize(r, 2, 16)
    assert z16[0, 0] > mn and q[0, 0] == 0


def test_overflowing_scale_is_rejected():
    r = np.zeros((1, 32), dtype=np.float32)
    r[0, 0], r[0, 1] = -2e5, 2e5
    with pytest.raises(OverflowError):
        codec.quantize(r, 2, 32)


# ------------------------------ packing ------------------------------

@pytest.mark.parametrize("bits", [2, 4])
def test_pack_every_code_at_every_position(bits):
    """Exhaustive: a single non-zero code lands at exactly one word and offset, and the
    offsets of all positions tile the words without overlap."""
    d = 128
    per = 32 // bits
    seen = np.zeros((d * bits // 32,), dtype=np.uint64)
    for i in range(d):
        for v in range(1, 1 << bits):
            q = np.zeros((1, d), dtype=np.uint8)
            q[0, i] = v
            w = codec.pack_codes(q, bits)[0]
            nz = np.flatnonzero(w)
            assert nz.tolist() == [i // per]
            assert int(w[i // per]) == v << (bits * (i % per))
            assert np.array_equal(codec.unpack_codes(w[None], bits, d), q)
        q = np.zeros((1, d), dtype=np.uint8)
        q[0, i] = (1 << bits) - 1
        w = codec.pack_codes(q, bits)[0].astype(np.uint64)
        assert np.all((seen & w) == 0)
        seen |= w
    assert np.all(seen == 0xFFFFFFFF)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_matches_string_construction(bits):
    """Independent construction: write each word as a binary string, highest element first."""
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 1 << bits, (20, 64)).astype(np.uint8)
    per = 32 // bits
    words = codec.pack_codes(q, bits)
    for r in range(q.shape[0]):
        for w in range(q.shape[1] // per):
            elems = q[r, w * per:(w + 1) * per]
            s = "".join(format(int(e), f"0{bits}b") for e in elems[::-1])
            assert int(words[r, w]) == int(s, 2)
    assert np.array_equal(codec.unpack_codes(words, bits, 64), q)


def test_scale_zero_word_and_index_dtype():
    s = np.array([1.0, 0.0], dtype=np.float16)
    z = np.array([-2.0, 0.25], dtype=np.float16)
    w = codec.pack_scale_zero(s, z)
    assert w.tolist() == [0xC0003C00, 0x34000000]
    s2, z2 = codec.unpack_scale_zero(w)
    assert np.array_equal(s2, s) and np.array_equal(z2, z)
    assert codec.index_dtype(256) == np.uint8 and codec.index_dtype(257) == np.uint16


def test_centroid_encode_store_layout_and_decode():
    rng = np.random.default_rng(7)
    n, h, d, k = 40, 3, 64, 10
    x = rng.standard_normal((n, h, d)).astype(np.float32)
    C = rng.standard_normal((h, k, d)).astype(np.float32)
    e = codec.encode_centroid(x, C, 4, 32)
    st = e["store"]
    assert st["codes"].shape == (h, n, d * 4 // 32) and st["codes"].dtype == np.uint32
    assert st["scale_zero"].shape == (h, n, d // 32)
    assert st["index"].shape == (h, n) and st["index"].dtype == np.uint8
    assert np.array_equal(st["index"].T, e["idx"])
    xhat = codec.decode_store(st, 4, 32, d, C=C)
    # reconstruction = centroid + dequantized residual, element by element
    base = C[np.arange(h)[None, :], e["idx"]]
    assert np.array_equal(xhat, base + codec.dequantize(e["q"], e["s16"], e["z16"], 32))
    # and lies within the quantizer's error bound of the input, group by group
    r = (x - base).reshape(n, h, 2, 32).astype(np.float64)
    s = e["s16"].astype(np.float64)
    z = e["z16"].astype(np.float64)
    mn, mx = r.min(-1), r.max(-1)
    bound = np.maximum.reduce([s / 2, z - mn, 15 * ((mx - mn) / 15 - s) + (mn - z)]) + 1e-5
    err = np.abs(xhat.astype(np.float64) - x).reshape(n, h, 2, 32).max(-1)
    assert np.all(err <= bound)
