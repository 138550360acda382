"""Seeded synthetic KV caches shaped like the video-DiT workloads on the pages.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the codec's or attention's arithmetic: the CPU oracle and the
HIP path both take their inputs from here and from nowhere else.

Recipes (readings of the workload descriptions; the pages publish no data):

* ``cluster`` tokens, per head: per-channel lognormal scales s_c = exp(0.5 N),
  two distinct outlier channels multiplied by 10, eight centres
  mu_j = s * N(0, 1), every token picks a centre uniformly and adds N(0, 0.1)
  noise ("N(0, v)" is read as standard deviation v).
* ``frames``: frame 0 is cluster tokens, frame t = 0.9 * frame t-1 + N(0, 0.3).
  1560 tokens per latent frame (832x480 at 16x spatial reduction per side).
* block-DPLR layer chain (cross-layer predictor of Coral-KV, Fig. 3): layer 0
  is cluster tokens, layer l applies the block-diagonal plus rank-r map to the
  true layer l-1 and adds N(0, 0.2).
* temporal AR(2) chain (TempoKV, Fig. 2b): per-channel AR(2) keys, values
  from the aligned key plus the previous value, Student-t (nu=4) innovations.

bf16 tensors are returned as ``uint16`` bit patterns; fp32 tensors as float32.
Every array is token-major ``[N][H][d]`` unless stated.
"""
from __future__ import annotations

import numpy as np

TOKENS_PER_FRAME = 1560


def rng_for(seed: int, *keys: int) -> np.random.Generator:
    """An independent stream for (seed, *keys); lets a caller regenerate a subset."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), *[int(k) for k in keys]]))


def bf16_bits(x) -> np.ndarray:
    """Round to bfloat16 (torch's RNE conversion) and return the raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


class ClusterProcess:
    """Per-head clustered token distribution (lognormal channel scales, 2 outliers x10)."""

    def __init__(self, rng: np.random.Generator, heads: int, dim: int, n_centers: int = 8,
                 noise: float = 0.1):
        self.heads, self.dim, self.n_centers, self.noise = heads, dim, n_centers, noise
        scales = np.exp(0.5 * rng.standard_normal((heads, dim)))
        for h in range(heads):
            out = rng.choice(dim, size=2, replace=False)
            scales[h, out] *= 10.0
        self.scales = scales
        self.centers = scales[:, None, :] * rng.standard_normal((heads, n_centers, dim))

    def draw(self, rng: np.random.Generator, n: int) -> np.ndarray:
        z = rng.integers(0, self.n_centers, size=(n, self.heads))
        x = self.centers[np.arange(self.heads)[None, :], z]  # [n, H, d]
        return x + self.noise * rng.standard_normal((n, self.heads, self.dim))


def frames(rng: np.random.Generator, proc: ClusterProcess, n_frames: int, tokens: int,
           rho: float = 0.9, sigma: float = 0.3) -> np.ndarray:
    """Frame 0 = cluster tokens; frame t = rho * frame t-1 + N(0, sigma). Returns [F*T, H, d]."""
    out = np.empty((n_frames * tokens, proc.heads, proc.dim), dtype=np.float64)
    cur = proc.draw(rng, tokens)
    out[:tokens] = cur
    for t in range(1, n_frames):
        cur = rho * cur + sigma * rng.standard_normal(cur.shape)
        out[t * tokens:(t + 1) * tokens] = cur
    return out


def sample_rows(rng: np.random.Generator, x: np.ndarray, count: int) -> np.ndarray:
    """Per head, `count` distinct history tokens: [N, H, d] -> [H, count, d]."""
    n, heads, _ = x.shape
    idx = np.stack([rng.choice(n, size=count, replace=False) for _ in range(heads)])
    return np.stack([x[idx[h], h] for h in range(heads)])


# ---------------------------------------------------------------------------
# Workload configurations
# ---------------------------------------------------------------------------

def cfg0(seed: int = 1234) -> dict:
    """Tiny centroid codec, fp32: 1 layer, 2 heads x 64, 256 history + 64 query tokens,
    16 centroids per head, INT4 residual, group 32, softmax scale 1/8."""
    rng = rng_for(seed, 0)
    heads, dim, n, nq, c = 2, 64, 256, 64, 16
    pk = ClusterProcess(rng, heads, dim)
    pv = ClusterProcess(rng, heads, dim)
    k = pk.draw(rng, n)
    v = pv.draw(rng, n)
    q = pk.draw(rng, nq)
    ck = sample_rows(rng, k, c)
    cv = sample_rows(rng, v, c)
    f = np.float32
    return dict(name="cfg0", dtype="f32", heads=heads, dim=dim, bits=4, group=32, centroids=c,
                K=k.astype(f), V=v.astype(f), Q=q.astype(f), Ck=ck.astype(f), Cv=cv.astype(f),
                scale=1.0 / 8.0)


def _video_centroid(seed: int, hist_frames: int, query_frames: int, tokens: int, heads: int,
                    dim: int, n_centroids: int) -> dict:
    rng = rng_for(seed, 0)
    pk = ClusterProcess(rng, heads, dim)
    pv = ClusterProcess(rng, heads, dim)
    kq = frames(rng_for(seed, 1), pk, hist_frames + query_frames, tokens)
    v = frames(rng_for(seed, 2), pv, hist_frames, tokens)
    nh = hist_frames * tokens
    k, q = kq[:nh], kq[nh:]
    crng = rng_for(seed, 3)
    ck = sample_rows(crng, k, n_centroids)
    cv = sample_rows(crng, v, n_centroids)
    return dict(heads=heads, dim=dim, tokens_per_frame=tokens, K=bf16_bits(k), V=bf16_bits(v),
                Q=bf16_bits(q), Ck=bf16_bits(ck), Cv=bf16_bits(cv), dtype="bf16",
                scale=1.0 / np.sqrt(dim))


def cfg1(seed: int = 1235, hist_frames: int = 21, query_frames: int = 3,
         tokens: int = TOKENS_PER_FRAME, heads: int = 12, dim: int = 128,
         n_centroids: int = 256) -> dict:
    """Centroid + INT2 (group 32) codec, bf16, one 1.3B-class layer (12 x 128).
    History 21 frames x 1560 = 32760 tokens; queries are the next 3 frames of the key
    process (4680); 256 centroids per head sampled from the history. The timed encode is
    the last 3-frame chunk of the history."""
    d = _video_centroid(seed, hist_frames, query_frames, tokens, heads, dim, n_centroids)
    chunk = 3 * tokens
    nh = hist_frames * tokens
    d.update(name="cfg1", bits=2, group=32, centroids=n_centroids,
             chunk=(max(0, nh - chunk), nh))
    return d


def cfg4(seed: int = 1238, hist_frames: int = 42, query_frames: int = 3,
         tokens: int = TOKENS_PER_FRAME, heads: int = 12, dim: int = 128,
         n_centroids: int = 512, coeff_dim: int = 16) -> dict:
    """Mixed-dimensional attention workload: 12 x 128, 42 frames x 1560 = 65520 keys,
    512 centroids per head, shared basis B = orthonormal (QR) d x m stored in bf16,
    INT4 key coefficients (group m), INT2 group-32 values, 4680 queries."""
    d = _video_centroid(seed, hist_frames, query_frames, tokens, heads, dim, n_centroids)
    g = rng_for(seed, 4).standard_normal((dim, coeff_dim))
    basis, _ = np.linalg.qr(g)
    d.update(name="cfg4", centroids=n_centroids, coeff_dim=coeff_dim, B=bf16_bits(basis),
             k_bits=4, k_group=coeff_dim, v_bits=2, v_group=32)
    return d


# --------------------------- block-DPLR layer chain ---------------------------

def cfg2_params(seed: int = 1236, heads: int = 12, dim: int = 128, rank: int = 64) -> dict:
    """Seeded near-identity block-diagonal blocks plus small low-rank factors, bf16 bits.

    WK [H][d][d], UK [D][r], VK [D][r]       (key map over K_{l-1})
    WV [H][d][2d], UV [D][r], VV [2D][r]     (value map over [K_l ; V_{l-1}])
    with D = H*d; the value low-rank input is [K_l (all heads) ; V_{l-1} (all heads)]."""
    rng = rng_for(seed, 100)
    D = heads * dim
    eye = np.eye(dim)
    wk = eye[None] + 0.05 * rng.standard_normal((heads, dim, dim)) / np.sqrt(dim)
    wv = np.concatenate([0.5 * eye, 0.5 * eye], axis=1)[None] \
        + 0.05 * rng.standard_normal((heads, dim, 2 * dim)) / np.sqrt(2 * dim)
    uk = 0.05 * rng.standard_normal((D, rank)) / np.sqrt(D)
    vk = 0.05 * rng.standard_normal((D, rank)) / np.sqrt(D)
    uv = 0.05 * rng.standard_normal((D, rank)) / np.sqrt(D)
    vv = 0.05 * rng.standard_normal((2 * D, rank)) / np.sqrt(2 * D)
    return dict(heads=heads, dim=dim, rank=rank, WK=bf16_bits(wk), UK=bf16_bits(uk),
                VK=bf16_bits(vk), WV=bf16_bits(wv), UV=bf16_bits(uv), VV=bf16_bits(vv))


def _bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (generator-side plumbing)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _per_head(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[n, h] = w[h] @ x[n, h] for x [n][H][k], w [H][d][k] (per-head matrix products)."""
    return np.stack([x[:, h] @ w[h].T for h in range(w.shape[0])], axis=1)


def cfg2_layers(seed: int = 1236, params: dict | None = None, n_tokens: int = 21 * TOKENS_PER_FRAME,
                n_layers: int = 30, chunk_ids=None, chunk: int = TOKENS_PER_FRAME,
                noise: float = 0.2):
    """Yield (K_l, V_l) as bf16 bits [n][H][d] for l = 0..n_layers-1.

    Tokens are generated in chunks of `chunk` tokens, each with its own random stream,
    so any subset of chunks (`chunk_ids`) reproduces exactly the same rows."""
    if params is None:
        params = cfg2_params(seed)
    heads, dim = params["heads"], params["dim"]
    wk, uk, vk = (_bits_to_f64(params[n]) for n in ("WK", "UK", "VK"))
    wv, uv, vv = (_bits_to_f64(params[n]) for n in ("WV", "UV", "VV"))
    n_chunks = (n_tokens + chunk - 1) // chunk
    ids = list(range(n_chunks)) if chunk_ids is None else list(chunk_ids)
    sizes = [min(chunk, n_tokens - c * chunk) for c in ids]
    proc_rng = rng_for(seed, 101)
    pk = ClusterProcess(proc_rng, heads, dim)
    pv = ClusterProcess(proc_rng, heads, dim)
    D = heads * dim
    k_prev = v_prev = None
    for layer in range(n_layers):
        ks, vs = [], []
        for j, (c, m) in enumerate(zip(ids, sizes)):
            rng = rng_for(seed, 200 + layer, c)
            if layer == 0:
                k = pk.draw(rng, m)
                v = pv.draw(rng, m)
            else:
                kp, vp = k_prev[j], v_prev[j]
                k = _per_head(kp, wk) \
                    + ((kp.reshape(m, D) @ vk) @ uk.T).reshape(m, heads, dim) \
                    + noise * rng.standard_normal((m, heads, dim))
                kv = np.concatenate([k, vp], axis=2)  # per head [K_l,h ; V_{l-1},h]
                lr_in = np.concatenate([k.reshape(m, D), vp.reshape(m, D)], axis=1)
                v = _per_head(kv, wv) \
                    + ((lr_in @ vv) @ uv.T).reshape(m, heads, dim) \
                    + noise * rng.standard_normal((m, heads, dim))
            ks.append(k)
            vs.append(v)
        k_prev, v_prev = ks, vs
        yield bf16_bits(np.concatenate(ks)), bf16_bits(np.concatenate(vs))


# --------------------------- temporal AR(2) chain ---------------------------

def cfg3(seed: int = 1237, n_frames: int = 16, query_frames: int = 3,
         tokens: int = TOKENS_PER_FRAME, heads: int = 40, dim: int = 128) -> dict:
    """Temporal predictor workload, 13B-class shape (40 x 128), 16 frames x 1560 tokens.

    K_t = a*K_{t-1} + b*K_{t-2} + 0.3*t4 with a_c ~ U(1.0, 1.2), b_c ~ U(-0.35, -0.25),
    frame 0 cluster tokens and K_{-1} := K_0.  V_t = M_h K_t + beta*V_{t-1} + 0.3*t4 with
    M_h = G/sqrt(d), beta_c ~ U(0.3, 0.7), V_{-1} := 0.  Queries are the next 3 frames of
    the key process.  Returns the generator's coefficients rounded to their storage types
    (a, b, beta fp32; M bf16) for the predictor to use."""
    rng = rng_for(seed, 0)
    proc = ClusterProcess(rng, heads, dim)
    a = rng.uniform(1.0, 1.2, size=(heads, dim)).astype(np.float32)
    b = rng.uniform(-0.35, -0.25, size=(heads, dim)).astype(np.float32)
    beta = rng.uniform(0.3, 0.7, size=(heads, dim)).astype(np.float32)
    m_bits = bf16_bits(rng.standard_normal((heads, dim, dim)) / np.sqrt(dim))
    m = _bits_to_f64(m_bits)
    total = n_frames + query_frames
    K = np.empty((total * tokens, heads, dim), dtype=np.float32)
    V = np.empty((n_frames * tokens, heads, dim), dtype=np.float32)
    k0 = proc.draw(rng_for(seed, 1, 0), tokens)
    k1, k2 = k0, k0  # K_{t-1}, K_{t-2}
    vprev = np.zeros_like(k0)
    for t in range(total):
        r = rng_for(seed, 1, t + 1)
        if t == 0:
            k = k0
        else:
            k = a * k1 + b * k2 + 0.3 * r.standard_t(4, size=k0.shape)
        K[t * tokens:(t + 1) * tokens] = k
        if t < n_frames:
            v = _per_head(k, m) + beta * vprev \
                + 0.3 * r.standard_t(4, size=k0.shape)
            V[t * tokens:(t + 1) * tokens] = v
            vprev = v
        k2, k1 = k1, k
    nh = n_frames * tokens
    return dict(name="cfg3", dtype="bf16", heads=heads, dim=dim, tokens_per_frame=tokens,
                n_frames=n_frames, K=bf16_bits(K[:nh]), V=bf16_bits(V), Q=bf16_bits(K[nh:]),
                a=a, b=b, beta=beta, M=m_bits, bits=2, group=64, anchor_bits=4,
                scale=1.0 / np.sqrt(dim))


def cfg2_layers_device(device, seed: int = 1236, params: dict | None = None,
                       n_tokens: int = 21 * TOKENS_PER_FRAME, n_layers: int = 30,
                       noise: float = 0.2):
    """The block-DPLR layer process of cfg2_layers drawn with torch's generator on
    `device` (full-size runs); yields (K_l, V_l) as bf16 tensors [n][H][d].  Same recipe,
    different random stream: use cfg2_layers where values must match the oracle's."""
    import torch

    if params is None:
        params = cfg2_params(seed)
    heads, dim = params["heads"], params["dim"]
    D = heads * dim

    def f(name):
        b = torch.from_numpy(params[name].view(np.int16)).view(torch.bfloat16)
        return b.to(device=device, dtype=torch.float32)

    wk, uk, vk, wv, uv, vv = (f(n) for n in ("WK", "UK", "VK", "WV", "UV", "VV"))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    proc = ClusterProcess(rng_for(seed, 101), heads, dim)
    centers = torch.from_numpy(proc.centers).to(device=device, dtype=torch.float32)

    def cluster(n):
        z = torch.randint(0, proc.n_centers, (n, heads), generator=gen, device=device)
        x = centers[torch.arange(heads, device=device)[None, :], z]
        return x + proc.noise * torch.randn((n, heads, dim), generator=gen, device=device)

    k = cluster(n_tokens)
    v = cluster(n_tokens)
    for layer in range(n_layers):
        if layer:
            kp, vp = k, v
            k = torch.einsum("hij,nhj->nhi", wk, kp).contiguous() + ((kp.reshape(-1, D) @ vk) @ uk.T).reshape(
                -1, heads, dim) + noise * torch.randn(kp.shape, generator=gen, device=device)
            kv = torch.cat([k, vp], dim=2)
            lr = torch.cat([k.reshape(-1, D), vp.reshape(-1, D)], dim=1)
            v = torch.einsum("hij,nhj->nhi", wv, kv).contiguous() + ((lr @ vv) @ uv.T).reshape(
                -1, heads, dim) + noise * torch.randn(vp.shape, generator=gen, device=device)
        yield k.to(torch.bfloat16).contiguous(), v.to(torch.bfloat16).contiguous()
