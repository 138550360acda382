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
