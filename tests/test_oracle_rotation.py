"""Pins for the Hn residual rotation oracle and the rotated codec: exact integer
matrix products, the fp64 product within the binary32 bound, self-inverse, the
exact round trip of residuals that lie on the quantization grid after rotation,
the codec's error bound, and attention in rotated coordinates."""
import numpy as np
import pytest
import scipy.linalg

from oracle import attention, codec, predict, rotation


def _popcount_matrix(n):
    """H_n entries (-1)^popcount(i & j), built without the recursion."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(bits % 2 == 0, 1, -1).astype(np.int64)


@pytest.mark.parametrize("n", rotation.WIDTHS)
def test_small_integers_rotate_exactly(n):
    # integers times a power of two: every binary32 sum in the recursion is exact,
    # so the result must equal the integer matrix product scaled by 1/sqrt(n)
    rng = np.random.default_rng(n)
    xi = rng.integers(-50, 51, size=(7, 2 * n)).astype(np.int64)
    y = rotation.rotate(xi.astype(np.float32), n)
    for Hm in (scipy.linalg.hadamard(n).astype(np.int64), _popcount_matrix(n)):
        want = np.concatenate([xi[:, g * n:(g + 1) * n] @ Hm.T for g in range(2)], axis=1)
        np.testing.assert_array_equal(y, (want / np.sqrt(n)).astype(np.float32))


@pytest.mark.parametrize("n", rotation.WIDTHS)
def test_random_inputs_within_binary32_bound_of_fp64_product(n):
    rng = np.random.default_rng(100 + n)
    x = (rng.standard_normal((200, 128)) * np.exp(rng.standard_normal((200, 1)))).astype(np.float32)
    y = rotation.rotate(x, n).astype(np.float64)
    Hm = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
    xg = x.astype(np.float64).reshape(200, 128 // n, n)
    want = np.einsum("ij,bgj->bgi", Hm, xg).reshape(200, 128)
    # log2(n) rounded stages, each off by at most 2^-24 of a partial sum bounded by sum |x|
    bound = np.log2(n) * 2.0 ** -24 * np.abs(xg).sum(-1) / np.sqrt(n)
    err = np.abs(y - want).reshape(200, 128 // n, n).max(-1)
    assert np.all(err <= 1.01 * bound + 1e-45)


@pytest.mark.parametrize("n", rotation.WIDTHS)
def test_rotation_is_its_own_inverse_and_keeps_norms(n):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    y = rotation.rotate(x, n)
    np.testing.assert_allclose(rotation.rotate(y, n), x, rtol=0, atol=1e-5)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    # a unit vector at channel 0 of a group spreads to a constant 1/sqrt(n) over that group only
    e = np.zeros((1, 128), np.float32)
    e[0, n] = 1
    ye = rotation.rotate(e, n)[0]
    assert np.all(ye[n:2 * n] == np.float32(1 / np.sqrt(n)))
    assert np.all(ye[:n] == 0) and np.all(ye[2 * n:] == 0)


def test_rotation_rejects_other_widths():
    with pytest.raises(ValueError):
        rotation.rotate(np.zeros((1, 128), np.float32), 32)
    with pytest.raises(ValueError):
        rotation.rotate(np.zeros((1, 48), np.float32), 64)


def _grid_case(n, bits, group, seed):
    """x = C[a] + H v with v on the quantizer's grid in every group (codes 0 and
    2^b - 1 present), small-integer multiples of 2^-5 so every operation is exact."""
    rng = np.random.default_rng(seed)
    N, H, K, d = 40, 2, 6, 128
    L = (1 << bits) - 1
    C = (rng.integers(-8, 9, size=(H, K, d)) * 4.0).astype(np.float32)      # far apart
    a = rng.integers(0, K, size=(N, H))
    codes = rng.integers(0, L + 1, size=(N, H, d // group, group))
    codes[..., 0] = 0
    codes[..., 1] = L
    s = 2.0 ** -rng.integers(2, 4, size=(N, H, d // group, 1))
    z = -rng.integers(0, 4, size=(N, H, d // group, 1)) * 2.0 ** -3
    v = (codes * s + z).reshape(N, H, d).astype(np.float32)
    base = C[np.arange(H)[None, :], a]
    x = base + rotation.rotate(v, n)
    return x.astype(np.float32), C, a, v


@pytest.mark.parametrize("n,bits,group", [(64, 2, 64), (16, 2, 64), (16, 4, 32), (16, 2, 16)])
def test_grid_residuals_round_trip_exactly_only_with_rotation(n, bits, group):
    x, C, a, v = _grid_case(n, bits, group, seed=n + bits + group)
    enc = codec.encode_centroid(x, C, bits, group, rotation=n)
    np.testing.assert_array_equal(enc["idx"], a)
    xh = codec.decode_store(enc["store"], bits, group, 128, C=C, rotation=n)
    np.testing.assert_array_equal(xh, x)
    # the same vectors through the unrotated codec are not reproduced
    plain = codec.encode_centroid(x, C, bits, group)
    xp = codec.decode_store(plain["store"], bits, group, 128, C=C)
    assert np.abs(xp - x).max() > 1e-3


@pytest.mark.parametrize("n,bits,group", [(64, 2, 64), (16, 2, 64), (64, 4, 64), (16, 4, 32)])
def test_rotated_codec_error_bound(n, bits, group):
    rng = np.random.default_rng(3)
    N, H, K, d = 300, 3, 16, 128
    C = rng.standard_normal((H, K, d)).astype(np.float32)
    x = (C[np.arange(H)[None, :], rng.integers(0, K, (N, H))]
         + 0.3 * rng.standard_normal((N, H, d))).astype(np.float32)
    enc = codec.encode_centroid(x, C, bits, group, rotation=n)
    xh = codec.decode_store(enc["store"], bits, group, d, C=C, rotation=n)
    s = enc["s16"].astype(np.float64)                       # [N, H, d/g]
    # the rotation keeps Euclidean norms, so the error norm is that of the rotated
    # residual's quantization error: at most s/2 per element (+ binary32 rounding)
    bound = np.sqrt((group * (s / 2) ** 2).sum(-1)) * (1 + 1e-5) + 1e-5
    err = np.linalg.norm((xh - x).astype(np.float64), axis=-1)
    assert np.all(err <= bound)


@pytest.mark.parametrize("nk,nv", [(64, 64), (16, 64), (64, 0)])
def test_attention_in_rotated_coordinates_matches_decoded_cache(nk, nv):
    # scores q . (c + H r') = (H q) . (H c + r') and O = H (sum p (H c_v + r'_v)):
    # attention with rotated queries and tables, output rotated back, is attention
    # over the decoded cache
    rng = np.random.default_rng(11)
    N, M, H, K, d, bits, group = 90, 17, 2, 8, 128, 2, 64
    Ck = rng.standard_normal((H, K, d)).astype(np.float32)
    Cv = rng.standard_normal((H, K, d)).astype(np.float32)
    kx = (Ck[np.arange(H)[None, :], rng.integers(0, K, (N, H))] + 0.4 * rng.standard_normal((N, H, d))).astype(np.float32)
    vx = (Cv[np.arange(H)[None, :], rng.integers(0, K, (N, H))] + 0.4 * rng.standard_normal((N, H, d))).astype(np.float32)
    q = rng.standard_normal((M, H, d)).astype(np.float32)
    ek = codec.encode_centroid(kx, Ck, bits, group, rotation=nk)
    ev = codec.encode_centroid(vx, Cv, bits, group, rotation=nv)
    kd = codec.decode_store(ek["store"], bits, group, d, C=Ck, rotation=nk)
    vd = codec.decode_store(ev["store"], bits, group, d, C=Cv, rotation=nv)
    want = attention.attention(q, kd, vd, 0.09)

    def rot64(a, n):          # exact fp64 rotation by the matrix
        if not n:
            return np.asarray(a, np.float64)
        Hm = scipy.linalg.hadamard(n) / np.sqrt(n)
        g = np.asarray(a, np.float64).reshape(*a.shape[:-1], d // n, n)
        return np.einsum("ij,...gj->...gi", Hm, g).reshape(a.shape)

    def deq(e, b):
        qd = np.transpose(codec.unpack_codes(e["store"]["codes"], b, d), (1, 0, 2))
        s16, z16 = codec.unpack_scale_zero(np.transpose(e["store"]["scale_zero"], (1, 0, 2)))
        return codec.dequantize(qd, s16, z16, group).astype(np.float64)

    kr = rot64(Ck, nk)[np.arange(H)[None, :], ek["idx"]] + deq(ek, bits)
    vr = rot64(Cv, nv)[np.arange(H)[None, :], ev["idx"]] + deq(ev, bits)
    got = rot64(attention.attention(rot64(q, nk), kr, vr, 0.09), nv)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-5)


@pytest.mark.parametrize("n,bits,group", [(64, 2, 64), (16, 2, 32), (16, 4, 16), (64, 4, 64)])
def test_prediction_residuals_rotated_grid_round_trip(n, bits, group):
    """The predictor path rotates the prediction residual: an input equal to the
    prediction plus H v, v on the quantizer's grid, is reconstructed exactly through
    the rotated codec and not through the plain one."""
    x, C, a, v = _grid_case(n, bits, group, seed=3 * n + bits + group)
    pred = C[np.arange(C.shape[0])[None, :], a].astype(np.float64)   # any fp32-exact base
    enc = predict.encode_with_prediction(x, pred, bits, group, rotation=n)
    np.testing.assert_array_equal(enc["xhat"], x)
    np.testing.assert_array_equal(
        codec.dequantize(enc["q"], enc["s16"], enc["z16"], group), v)
    plain = predict.encode_with_prediction(x, pred, bits, group)
    assert np.abs(plain["xhat"] - x).max() > 1e-3


@pytest.mark.parametrize("n,bits,group", [(64, 2, 64), (16, 2, 32)])
def test_rotated_dplr_chain_error_bound(n, bits, group):
    """Each predicted layer of a rotated cross-layer chain keeps the rotated
    quantizer's error bound: |x - x_hat| <= sqrt(sum over groups of g (s/2)^2)."""
    rng = np.random.default_rng(8)
    h, d, r, N, L = 2, 128, 8, 30, 3
    WK = np.broadcast_to(np.eye(d), (h, d, d)) + 0.05 * rng.standard_normal((h, d, d))
    WV = np.concatenate([0.5 * np.eye(d)] * 2, 1)[None] + 0.05 * rng.standard_normal((h, d, 2 * d))
    params = dict(WK=WK, UK=0.05 * rng.standard_normal((h * d, r)), VK=0.05 * rng.standard_normal((h * d, r)),
                  WV=WV, UV=0.05 * rng.standard_normal((h * d, r)), VV=0.05 * rng.standard_normal((2 * h * d, r)))
    layers = [(rng.standard_normal((N, h, d)).astype(np.float32),
               rng.standard_normal((N, h, d)).astype(np.float32)) for _ in range(L)]
    outs = list(predict.dplr_chain(layers, params, bits, group, 4, anchor_group=32, rotation=n))
    for (k, v), o in zip(layers[1:], outs[1:]):
        for x, e in ((k, o["k"]), (v, o["v"])):
            s = e["s16"].astype(np.float64)
            bound = np.sqrt((group * (s / 2) ** 2).sum(-1)) * (1 + 1e-5) + 1e-5
            err = np.linalg.norm((e["xhat"] - x).astype(np.float64), axis=-1)
            assert np.all(err <= bound)
