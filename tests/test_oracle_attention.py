"""Pins for the attention oracle: torch's fp64 SDPA (library routine), closed-form
special cases, a hand-worked example, and the mixed-dimensional identity."""
import math

import numpy as np
import torch

from oracle import attention, coeff, codec, numerics as nm


def test_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((37, 3, 16)) * 2
    k = rng.standard_normal((101, 3, 16)) * 2
    v = rng.standard_normal((101, 3, 16))
    scale = 0.3
    out = attention.attention(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2))) for a in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
    assert np.allclose(out, want.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_hand_worked_example():
    # logits 0 and ln 3 -> weights 1/4, 3/4; O = 1/4 (4, 0) + 3/4 (0, 8) = (1, 6)
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[0.0, 0.0]], [[math.log(3.0), 0.0]]])
    v = np.array([[[4.0, 0.0]], [[0.0, 8.0]]])
    out, lse = attention.attention(q, k, v, 1.0, return_lse=True)
    assert np.allclose(out[0, 0], [1.0, 6.0], atol=1e-14)
    assert np.isclose(lse[0, 0], math.log(4.0))


def test_single_key_and_zero_query():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    q = rng.standard_normal((5, 2, 8))
    assert np.allclose(attention.attention(q, k, v, 0.5), np.broadcast_to(v, (5, 2, 8)))
    k = rng.standard_normal((50, 2, 8))
    v = rng.standard_normal((50, 2, 8))
    out = attention.attention(np.zeros((3, 2, 8)), k, v, 0.5)
    assert np.allclose(out, np.broadcast_to(v.mean(0), (3, 2, 8)), atol=1e-14)


def test_cache_view_rounds_bf16_only():
    x = np.array([1 + 2.0 ** -9, 3.14159], dtype=np.float32)
    assert np.array_equal(attention.cache_view(x, "f32"), x)
    assert np.array_equal(attention.cache_view(x, "bf16"), nm.round_bf16(x))


def test_mixed_dimensional_identity():
    """(q . C[a] + (B^T q) . c) * scale == q . (C[a] + B c) * scale."""
    rng = np.random.default_rng(2)
    h, d, m, nk, nq, C = 2, 32, 8, 200, 9, 12
    B, _ = np.linalg.qr(rng.standard_normal((d, m)))
    B = nm.round_bf16(B.astype(np.float32))
    k = rng.standard_normal((nk, h, d)).astype(np.float32)
    Ck = rng.standard_normal((h, C, d)).astype(np.float32)
    e = coeff.encode_coeff(k, Ck, B, 4)
    q = rng.standard_normal((nq, h, d))
    s = attention.mixed_scores(q, Ck, e["idx"], B, e["chat"], 0.25)
    khat = coeff.reconstruct_keys(Ck, e["idx"], B, e["chat"])
    want = np.einsum("qhd,khd->hqk", q, khat) * 0.25
    assert np.allclose(s, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    vv = rng.standard_normal((nk, h, d))
    assert np.allclose(attention.mixed_attention(q, Ck, e["idx"], B, e["chat"], vv, 0.25),
                       attention.attention(q, khat, vv, 0.25), atol=1e-12)


def test_mixed_with_identity_basis_equals_centroid_codec_attention():
    """m = d, B = I: the coefficient codec is the centroid codec with group d, and the
    mixed-dimensional scores equal dense attention on the decoded keys."""
    rng = np.random.default_rng(3)
    h, d, nk, nq, C = 2, 16, 64, 5, 6
    k = rng.standard_normal((nk, h, d)).astype(np.float32)
    Ck = rng.standard_normal((h, C, d)).astype(np.float32)
    B = np.eye(d, dtype=np.float32)
    e = coeff.encode_coeff(k, Ck, B, 4)
    ec = codec.encode_centroid(k, Ck, 4, d)
    assert np.array_equal(e["store"]["codes"], ec["store"]["codes"])
    assert np.array_equal(e["store"]["scale_zero"], ec["store"]["scale_zero"])
    khat = codec.decode_store(ec["store"], 4, d, d, C=Ck)
    q = rng.standard_normal((nq, h, d))
    v = rng.standard_normal((nk, h, d))
    assert np.allclose(attention.mixed_attention(q, Ck, e["idx"], B, e["chat"], v, 0.3),
                       attention.attention(q, khat, v, 0.3), atol=1e-12)


def test_chunk_attention_is_the_lse_merge_of_its_parts():
    """One softmax over [history; chunk] equals the two parts' attentions weighted by
    exp(lse_part - lse) (flash-attention's split merge), and the merged lse is the
    log of the summed exponentials; brute force on a tiny case checks one output."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((7, 2, 16))
    kh, vh = rng.standard_normal((11, 2, 16)), rng.standard_normal((11, 2, 16))
    kc, vc = rng.standard_normal((3, 2, 16)) * 2.0, rng.standard_normal((3, 2, 16))
    out, lse = attention.attention_with_chunk(q, kh, vh, kc, vc, 0.3, return_lse=True)
    o1, l1 = attention.attention(q, kh, vh, 0.3, return_lse=True)
    o2, l2 = attention.attention(q, kc, vc, 0.3, return_lse=True)
    w1 = np.exp(l1 - lse).T[..., None]   # [nq, H, 1]
    w2 = np.exp(l2 - lse).T[..., None]
    assert np.allclose(w1 + w2, 1.0, atol=1e-12)
    assert np.allclose(out, w1 * o1 + w2 * o2, atol=1e-12)
    assert np.allclose(lse, np.logaddexp(l1, l2), atol=1e-12)
    # brute force: query 4, head 1
    s = [float(q[4, 1] @ k) * 0.3 for k in np.concatenate([kh, kc])[:, 1]]
    p = np.exp(np.array(s) - max(s))
    ref = (p[:, None] * np.concatenate([vh, vc])[:, 1]).sum(0) / p.sum()
    assert np.allclose(out[4, 1], ref, atol=1e-12)


# ------------------------------ Jensen-bias correction ------------------------------

def test_jensen_correction_is_the_second_order_term_of_uniform_noise():
    # for e uniform on [-s/2, s/2]: log E[exp(a e)] = log(sinh(x) / x), x = a s / 2,
    # = x^2 / 6 - x^4 / 180 + ...; the correction must be the x^2 / 6 term summed over
    # channels, so it agrees with the exact value to within the x^4 term
    rng = np.random.default_rng(5)
    nq, nk, H, d, g = 7, 9, 2, 64, 16
    q = rng.standard_normal((nq, H, d))
    step = rng.uniform(0.01, 0.3, size=(nk, H, d // g))
    scale = 0.125
    corr = attention.jensen_correction(q, step, g, scale)
    s_ch = np.repeat(step, g, axis=-1)                                   # [nk,H,d]
    for h in range(H):
        x = scale * q[:, h, None, :] * s_ch[None, :, h, :] / 2           # [nq,nk,d]
        exact = np.where(x == 0, 0.0, np.log(np.sinh(x) / np.where(x == 0, 1, x))).sum(-1)
        fourth = (x ** 4).sum(-1) / 180
        assert np.all(np.abs(corr[h] - exact) <= 1.01 * fourth + 1e-15)
        assert np.all(np.abs(corr[h] - exact) <= 0.05 * corr[h] + 1e-15)


def test_jensen_corrected_weights_are_unbiased_by_monte_carlo():
    # noisy keys k + e, e uniform with the per-group steps: the mean of exp(logit - corr)
    # recovers exp(logit of k) within Monte Carlo error, the plain mean does not
    rng = np.random.default_rng(6)
    d, g, scale = 32, 16, 0.25
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    step = np.array([[[0.8, 1.2]]])
    corr = attention.jensen_correction(q, step, g, scale)[0, 0, 0]
    s_ch = np.repeat(step[0, 0], g)
    e = (rng.random((400000, d)) - 0.5) * s_ch
    logits = scale * ((k[0, 0] + e) @ q[0, 0])
    true = scale * float(k[0, 0] @ q[0, 0])
    w = np.exp(logits - true)
    sem = w.std() / np.sqrt(w.size)
    assert abs(np.exp(-corr) * w.mean() - 1.0) < 4 * sem + 2e-4
    assert w.mean() - 1.0 > 20 * sem                   # the bias the correction removes


def test_jensen_attention_reduces_to_plain_and_chunk_forms():
    rng = np.random.default_rng(7)
    nq, nk, nc, H, d, g = 5, 11, 4, 2, 32, 16
    q, k, v = (rng.standard_normal((n, H, d)) for n in (nq, nk, nk))
    kc, vc = rng.standard_normal((nc, H, d)), rng.standard_normal((nc, H, d))
    zero = np.zeros((nk, H, d // g))
    np.testing.assert_allclose(attention.attention_jensen(q, k, v, zero, g, 0.3),
                               attention.attention(q, k, v, 0.3), rtol=0, atol=1e-12)
    np.testing.assert_allclose(
        attention.attention_jensen(q, k, v, zero, g, 0.3, k_chunk=kc, v_chunk=vc),
        attention.attention_with_chunk(q, k, v, kc, vc, 0.3), rtol=0, atol=1e-12)
    # a uniform step on every key shifts all history logits of a query by the same
    # amount: with no chunk the softmax is unchanged, with a chunk the history's total
    # weight drops by exactly exp(-corr)
    step = np.full((nk, H, d // g), 0.5)
    np.testing.assert_allclose(attention.attention_jensen(q, k, v, step, g, 0.3),
                               attention.attention(q, k, v, 0.3), rtol=0, atol=1e-12)
    corr = attention.jensen_correction(q, step, g, 0.3)[:, :, 0]          # [H, nq]
    _, lse_h = attention.attention(q, k, v, 0.3, return_lse=True)
    _, lse_c = attention.attention(q, kc, vc, 0.3, return_lse=True)
    _, lse = attention.attention_jensen(q, k, v, step, g, 0.3, k_chunk=kc, v_chunk=vc,
                                        return_lse=True)
    np.testing.assert_allclose(lse, np.logaddexp(lse_h - corr, lse_c), rtol=0, atol=1e-12)
