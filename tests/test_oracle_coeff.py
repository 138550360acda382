"""Pins for the coefficient oracle: identity basis, span reconstruction, fp64 bound."""
import numpy as np

from oracle import coeff, codec


def test_identity_basis_gives_residual_bitwise():
    rng = np.random.default_rng(0)
    r = rng.standard_normal((30, 2, 16)).astype(np.float32)
    c = coeff.coefficients(r, np.eye(16, dtype=np.float32))
    assert np.array_equal(c, r)


def test_fixed_order_sum_within_fp32_bound_of_fp64_product():
    rng = np.random.default_rng(1)
    d, m = 128, 16
    r = (rng.standard_normal((200, 3, d)) * 5).astype(np.float32)
    B = rng.standard_normal((d, m)).astype(np.float32)
    c = coeff.coefficients(r, B).astype(np.float64)
    exact = r.astype(np.float64) @ B.astype(np.float64)
    bound = d * 2.0 ** -24 * (np.abs(r).astype(np.float64) @ np.abs(B).astype(np.float64))
    assert np.all(np.abs(c - exact) <= bound)
    # and the order is ascending: recompute one entry step by step
    acc = np.float32(0)
    for i in range(d):
        acc = np.float32(acc + np.float32(r[7, 1, i] * B[i, 5]))
    assert acc == np.float32(c[7, 1, 5])


def test_residual_in_span_is_recovered():
    rng = np.random.default_rng(2)
    d, m = 64, 8
    B, _ = np.linalg.qr(rng.standard_normal((d, m)))
    B = B.astype(np.float32)
    w = rng.standard_normal((50, 2, m))
    Ck = rng.standard_normal((2, 4, d)).astype(np.float32)
    # keys = a centroid + B w; with 4 well separated centroids the assignment is that centroid
    Ck *= 20
    a = rng.integers(0, 4, (50, 2))
    k = (Ck[np.arange(2)[None, :], a] + (w @ B.T.astype(np.float64))).astype(np.float32)
    e = coeff.encode_coeff(k, Ck, B, 4)
    assert np.array_equal(e["idx"], a)
    assert np.allclose(e["coeff"], w, atol=1e-4 * 20)
    # dequantized coefficients within half a scale of the exact ones
    s = e["s16"].astype(np.float32)
    assert np.all(np.abs(e["chat"] - e["coeff"]) <= s / 2 + 1e-5 + np.abs(e["z16"].astype(np.float32) - e["coeff"].min(-1, keepdims=True)))
    khat = coeff.reconstruct_keys(Ck, e["idx"], B, e["chat"])
    assert np.abs(khat - k).max() <= np.sqrt(m) * s.max()
