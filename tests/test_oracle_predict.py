"""Pins for the predictor oracle: DPCM special cases, dense-matrix and brute-force
equivalence of the block-DPLR map, and chain error bounds."""
import numpy as np

from oracle import predict, numerics as nm


def _params(rng, h, d, r, n_in, scale=0.3):
    D = h * d
    return (rng.standard_normal((h, d, n_in * d)) * scale, rng.standard_normal((D, r)) * scale,
            rng.standard_normal((n_in * D, r)) * scale)


def test_dplr_identity_is_previous_layer():
    rng = np.random.default_rng(0)
    h, d, r = 3, 8, 2
    x = rng.standard_normal((20, h, d)).astype(np.float32)
    W = np.broadcast_to(np.eye(d), (h, d, d))
    out = predict.dplr_predict([x], W, np.zeros((h * d, r)), rng.standard_normal((h * d, r)))
    assert np.array_equal(out, nm.round_bf16(x).astype(np.float64))


def test_dplr_equals_dense_matrix_and_brute_force():
    rng = np.random.default_rng(1)
    h, d, r = 2, 4, 3
    for n_in in (1, 2):
        W, U, V = _params(rng, h, d, r, n_in)
        xs = [rng.standard_normal((6, h, d)).astype(np.float32) for _ in range(n_in)]
        out = predict.dplr_predict(xs, W, U, V)
        xb = [nm.round_bf16(x).astype(np.float64) for x in xs]
        xlr = np.concatenate([x.reshape(6, h * d) for x in xb], axis=1)
        dense = predict.dplr_dense_matrix(W, U, V, n_in)
        assert np.allclose(out.reshape(6, h * d), xlr @ dense.T, rtol=1e-12, atol=1e-12)
        # brute force from the definition, one output at a time
        for n in range(6):
            for hh in range(h):
                for i in range(d):
                    acc = 0.0
                    for j in range(n_in):
                        for c in range(d):
                            acc += W[hh, i, j * d + c] * xb[j][n, hh, c]
                    for kk in range(r):
                        t = 0.0
                        for l in range(n_in * h * d):
                            t += V[l, kk] * xlr[n, l]
                        acc += U[hh * d + i, kk] * t
                    assert abs(acc - out[n, hh, i]) <= 1e-12 * (1 + abs(acc))


def test_temporal_k_special_cases_and_order():
    rng = np.random.default_rng(2)
    k1 = rng.standard_normal((10, 2, 8)).astype(np.float32)
    k2 = rng.standard_normal((10, 2, 8)).astype(np.float32)
    one, zero = np.ones((2, 8), np.float32), np.zeros((2, 8), np.float32)
    assert np.array_equal(predict.temporal_predict_k(k1, k2, one, zero), nm.round_bf16(k1))
    a = rng.uniform(1, 1.2, (2, 8)).astype(np.float32)
    b = rng.uniform(-0.35, -0.25, (2, 8)).astype(np.float32)
    got = predict.temporal_predict_k(k1, k2, a, b)
    x1, x2 = nm.round_bf16(k1), nm.round_bf16(k2)
    for idx in [(0, 0, 0), (3, 1, 7), (9, 0, 4)]:
        want = np.float32(np.float32(a[idx[1:]] * x1[idx]) + np.float32(b[idx[1:]] * x2[idx]))
        assert got[idx] == want


def test_temporal_v_special_cases():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((10, 2, 8)).astype(np.float32)
    v = rng.standard_normal((10, 2, 8)).astype(np.float32)
    beta = rng.uniform(0.3, 0.7, (2, 8)).astype(np.float32)
    out = predict.temporal_predict_v(k, v, np.zeros((2, 8, 8)), beta)
    assert np.allclose(out, beta.astype(np.float64) * nm.round_bf16(v), rtol=1e-15)
    out = predict.temporal_predict_v(k, v, np.broadcast_to(np.eye(8), (2, 8, 8)), np.zeros((2, 8)))
    assert np.array_equal(out, nm.round_bf16(k).astype(np.float64))


def test_temporal_v_per_element_brute_force():
    """Each predicted value, summed term by term in exact rational arithmetic: channel i of
    head h is sum_j M[h, i, j] * bf16(K_t)[h, j] + beta[h, i] * bf16(V_{t-1})[h, i].  M_h
    is non-symmetric, so a transposed M_h (or a mixed-up head) fails."""
    from fractions import Fraction
    rng = np.random.default_rng(31)
    n, h, d = 5, 3, 8
    k = rng.standard_normal((n, h, d)).astype(np.float32)
    v = rng.standard_normal((n, h, d)).astype(np.float32)
    M = rng.standard_normal((h, d, d)) / np.sqrt(d)
    assert np.abs(M - M.transpose(0, 2, 1)).max() > 0.1
    beta = rng.uniform(0.3, 0.7, (h, d)).astype(np.float32)
    got = predict.temporal_predict_v(k, v, M, beta)
    kb, vb = nm.round_bf16(k), nm.round_bf16(v)
    for t in range(n):
        for hh in range(h):
            for i in range(d):
                exact = sum(Fraction(float(M[hh, i, j])) * Fraction(float(kb[t, hh, j]))
                            for j in range(d))
                exact += Fraction(float(beta[hh, i])) * Fraction(float(vb[t, hh, i]))
                assert abs(got[t, hh, i] - float(exact)) <= 1e-13 * (1 + abs(float(exact)))
    # the transposed map gives a different prediction
    assert np.abs(predict.temporal_predict_v(k, v, M.transpose(0, 2, 1), beta) - got).max() > 1e-3


def test_temporal_chain_first_frame_uses_the_anchor_twice():
    """At t = 1 there is no K_{-1}: the key predictor reads the anchor frame's reconstruction
    for both terms, (a * K^_0) + (b * K^_0) in fp32; at t = 2 it reads K^_1 and K^_0.  With
    b != 0 this differs from taking K_{-1} as zero."""
    rng = np.random.default_rng(32)
    T, h, d = 6, 2, 64
    ks = [rng.standard_normal((T, h, d)).astype(np.float32) for _ in range(3)]
    vs = [rng.standard_normal((T, h, d)).astype(np.float32) for _ in range(3)]
    a = rng.uniform(1.0, 1.2, (h, d)).astype(np.float32)
    b = rng.uniform(-0.35, -0.25, (h, d)).astype(np.float32)
    M = rng.standard_normal((h, d, d)) / np.sqrt(d)
    beta = rng.uniform(0.3, 0.7, (h, d)).astype(np.float32)
    outs = list(predict.temporal_chain(ks, vs, a, b, M, beta, 2, 64, 4))
    k0 = nm.round_bf16(outs[0]["k"]["xhat"])
    k1 = nm.round_bf16(outs[1]["k"]["xhat"])
    for t, (x1, x2) in ((1, (k0, k0)), (2, (k1, k0))):
        base = outs[t]["k"]["base"]
        for idx in [(0, 0, 0), (2, 1, 17), (5, 0, 63), (3, 1, 40)]:
            want = np.float32(np.float32(a[idx[1:]] * x1[idx]) + np.float32(b[idx[1:]] * x2[idx]))
            assert base[idx] == want, (t, idx)
    zero_prev = (a * k0).astype(np.float32)
    assert np.abs(outs[1]["k"]["base"] - zero_prev).max() > 0.1


def _group_bound(x, xhat, st_q, s16, z16, bits, group):
    """Max |x - xhat| per group against the quantizer bound (see the codec tests)."""
    L = (1 << bits) - 1
    n, h, d = x.shape
    err = np.abs(xhat.astype(np.float64) - x).reshape(n, h, d // group, group).max(-1)
    s = s16.astype(np.float64)
    return err, s


def test_dplr_chain_reconstructs_within_quantization_error():
    rng = np.random.default_rng(4)
    h, d, r, n, L = 2, 32, 4, 40, 5
    WK = np.broadcast_to(np.eye(d), (h, d, d)) + 0.05 * rng.standard_normal((h, d, d))
    WV = np.concatenate([0.5 * np.eye(d)] * 2, 1)[None] + 0.05 * rng.standard_normal((h, d, 2 * d))
    params = dict(WK=nm.round_bf16(WK.astype(np.float32)), UK=0.05 * rng.standard_normal((h * d, r)),
                  VK=0.05 * rng.standard_normal((h * d, r)), UV=0.05 * rng.standard_normal((h * d, r)),
                  VV=0.05 * rng.standard_normal((2 * h * d, r)), WV=nm.round_bf16(WV.astype(np.float32)))
    layers = [(rng.standard_normal((n, h, d)).astype(np.float32),
               rng.standard_normal((n, h, d)).astype(np.float32)) for _ in range(L)]
    outs = list(predict.dplr_chain(layers, params, 2, 16, 4))
    for (k, v), o in zip(layers, outs):
        for x, e in ((k, o["k"]), (v, o["v"])):
            g = 16
            err = np.abs(e["xhat"].astype(np.float64) - x).reshape(n, h, d // g, g).max(-1)
            rr = (x - e["base"]).reshape(n, h, d // g, g).astype(np.float64)
            bits = 4 if o["layer"] == 0 else 2
            Lq = (1 << bits) - 1
            s, z = e["s16"].astype(np.float64), e["z16"].astype(np.float64)
            mn, mx = rr.min(-1), rr.max(-1)
            bound = np.maximum.reduce([s / 2, z - mn, Lq * ((mx - mn) / Lq - s) + (mn - z)])
            assert np.all(err <= bound + 1e-5 * (1 + np.abs(x).max()))
    # teacher forcing with the chain's own reconstructions reproduces the free-running chain
    teacher = [(o["k"]["xhat"], o["v"]["xhat"]) for o in outs]
    outs2 = list(predict.dplr_chain(layers, params, 2, 16, 4, teacher=teacher))
    for a, b in zip(outs, outs2):
        assert np.array_equal(a["k"]["store"]["codes"], b["k"]["store"]["codes"])


def test_temporal_chain_exact_dpcm_on_constant_frames():
    """a = 1, b = 0, M = 0, beta = 1 and identical frames: after the anchor, every residual is
    the anchor's reconstruction error, which the chain keeps re-coding within the bound."""
    rng = np.random.default_rng(5)
    f = rng.standard_normal((12, 2, 64)).astype(np.float32)
    frames = [f] * 4
    one, zero = np.ones((2, 64), np.float32), np.zeros((2, 64), np.float32)
    outs = list(predict.temporal_chain(frames, frames, one, zero, np.zeros((2, 64, 64)), one,
                                       2, 64, 4))
    for o in outs[1:]:
        assert np.array_equal(o["k"]["base"], nm.round_bf16(outs[o["frame"] - 1]["k"]["xhat"]))
