"""Pins for the online centroid fitting oracle (Lloyd iterations at block fill)."""
import numpy as np

from oracle import fit, numerics as nm


def _blobs(seed, heads=2, k=5, per=30, d=16, spread=0.05):
    rng = np.random.default_rng(seed)
    centers = rng.standard_normal((heads, k, d)) * 10
    labels = np.tile(np.arange(k).repeat(per), (heads, 1)).T              # [N, H]
    x = np.empty((k * per, heads, d), np.float32)
    for h in range(heads):
        x[:, h] = centers[h][labels[:, h]] + spread * rng.standard_normal((k * per, d))
    return nm.round_bf16(x), labels


def test_separated_blobs_reach_their_rounded_means_in_one_step():
    x, labels = _blobs(1)
    k = 5
    C0 = nm.round_bf16(np.stack([x[labels[:, h].searchsorted(np.arange(k)), h]
                                 for h in range(x.shape[1])]))           # one seed per blob
    C1, idx, counts = fit.lloyd_step(x, C0)
    assert np.array_equal(idx, labels)
    assert np.all(counts == 30)
    for h in range(x.shape[1]):
        for j in range(k):
            want = nm.round_bf16(x[labels[:, h] == j, h].astype(np.float64).mean(0).astype(np.float32))
            assert np.array_equal(C1[h, j], want)
    # a second step changes nothing: the fixed point
    C2, idx2, _ = fit.lloyd_step(x, C1)
    assert np.array_equal(idx2, labels) and np.array_equal(C2, C1)


def test_duplicate_centroid_stays_empty_and_one_centroid_is_the_mean():
    x, _ = _blobs(2, heads=1, k=3)
    C0 = nm.round_bf16(np.stack([x[0, 0], x[0, 0], x[40, 0], x[80, 0]])[None])
    C1, idx, counts = fit.lloyd_step(x, C0)
    assert counts[0, 1] == 0 and np.array_equal(C1[0, 1], C0[0, 1])   # ties go to index 0
    assert not np.any(idx[:, 0] == 1)
    C1, idx, counts = fit.lloyd_step(x, C0[:, :1])
    assert counts[0, 0] == x.shape[0]
    assert np.array_equal(C1[0, 0], nm.round_bf16(x[:, 0].astype(np.float64).mean(0).astype(np.float32)))


def test_each_step_satisfies_its_definition_and_the_objective_does_not_grow():
    rng = np.random.default_rng(3)
    N, H, K, d = 400, 2, 12, 32
    x = nm.round_bf16((rng.standard_normal((N, H, d)) * np.exp(rng.standard_normal((1, 1, d)))).astype(np.float32))
    C = nm.round_bf16(x[::N // K][:K].transpose(1, 0, 2).copy())
    prev = fit.objective(x, C)
    for _ in range(6):
        Cn, idx, counts = fit.lloyd_step(x, C)
        # brute force: fp64 nearest (gaps are far from fp32 ties here) and plain means
        dist = ((x.astype(np.float64)[:, :, None, :] - C.astype(np.float64)[None]) ** 2).sum(-1)
        assert np.array_equal(idx, dist.argmin(-1))
        for h in range(H):
            for j in range(K):
                m = idx[:, h] == j
                if m.any():
                    assert np.abs(Cn[h, j] - x[m, h].astype(np.float64).mean(0)).max() <= \
                        2.0 ** -8 * np.abs(x[m, h]).max() + 1e-30
                else:
                    assert np.array_equal(Cn[h, j], C[h, j])
        cur = fit.objective(x, Cn)
        # exact means never raise the objective; bf16 rounding of the centroids adds at
        # most sum of count * |rounding|^2 + the cross term, bounded loosely here
        slack = sum(counts[h, j] * float(np.sum((2.0 ** -8 * np.abs(Cn[h, j])) ** 2))
                    for h in range(H) for j in range(K)) * 4
        assert cur <= prev + slack
        prev, C = cur, Cn


def test_mean_rounds_to_fp32_then_to_bf16():
    """Worked example of the rounding the update takes: the exact mean rounded to fp32,
    then to bf16 (nearest even at each step).  Four tokens whose channel 0 holds 2, 2,
    2^-6 and 2^-28 (all bf16 values) have the exact mean 1 + 2^-8 + 2^-30.  In fp32 the
    2^-30 is lost (half an ulp at 1 is 2^-24), leaving 1 + 2^-8, the midpoint between the
    bf16 neighbours 1 and 1 + 2^-7, which ties to even: 1.  Rounding the exact mean to
    bf16 in one step would give 1 + 2^-7.  Channel 1 is the control against truncation:
    its mean 1.75 + 3 * 2^-9 is exact in fp32 and above the midpoint 1.75 + 2^-8, so it
    rounds up to 1.7578125."""
    x = np.zeros((4, 1, 16), np.float32)
    x[:, 0, 0] = [2.0, 2.0, 2.0 ** -6, 2.0 ** -28]
    x[:, 0, 1] = [1.75, 1.75, 1.75, 1.75 + 3 * 2.0 ** -7]
    assert np.array_equal(nm.round_bf16(x), x)                  # bf16 inputs
    C0 = np.zeros((1, 1, 16), np.float32)                       # one centroid: all tokens
    C1, idx, counts = fit.lloyd_step(x, C0)
    assert counts[0, 0] == 4 and np.all(idx == 0)
    assert C1[0, 0, 0] == 1.0                                   # fp32 tie -> even
    assert C1[0, 0, 1] == 1.7578125                             # above the midpoint -> up
    assert np.all(C1[0, 0, 2:] == 0.0)
