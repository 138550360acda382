"""The paired chunk encode (kvc_encode_kv: the keys and the values of one chunk, one
launch where the 16-token-wave centroid encoder serves the codec) against two kvc_encode
calls: the same stores, word for word, and rows outside the written range untouched;
the stores also match the oracle's."""
import numpy as np
import pytest
import torch

import kv_cache_compression_02_amd as kvc
import synth
from oracle import numerics as nm
from gpu_util import check_centroid_store, device, fill_sentinel, store_np, to_dev

pytestmark = pytest.mark.gpu


def _pair_vs_single(codec, d, dev, kb, vb, off, n, cap):
    K, V = to_dev(d["K"][:n], dev), to_dev(d["V"][:n], dev)
    pk, pv, sk, sv = (kvc.Store.allocate(codec, cap, dev) for _ in range(4))
    for st in (pk, pv, sk, sv):
        fill_sentinel(st)
    kvc.kvc_encode_kv(codec, K, V, pk, pv, off, kb, vb)
    kvc.kvc_encode(codec, K, sk, off, kb)
    kvc.kvc_encode(codec, V, sv, off, vb)
    torch.cuda.synchronize()
    for a, b in ((pk, sk), (pv, sv)):
        ga, gb = store_np(a), store_np(b)
        for key in ga:
            assert np.array_equal(ga[key], gb[key]), key
    return store_np(pk), store_np(pv)


@pytest.mark.parametrize("bits,group,C,rot", [(2, 32, 40, 0), (4, 16, 300, 0), (2, 64, 40, 64),
                                              (4, 32, 256, 16)])
def test_paired_centroid_encode_matches_two_calls_and_oracle(bits, group, C, rot):
    """300 tokens at row offset 7 of a 320-row store (a ragged tile; 300 centroids: the
    512-row table variant)."""
    dev = device()
    d = synth.cfg1(seed=41, hist_frames=3, query_frames=1, tokens=100, heads=3, dim=128,
                   n_centroids=C)
    codec = kvc.Codec(3, 128, bits, group, kvc.BASE_CENTROID, C, rotation=rot)
    kb = kvc.BaseParams(centroids=to_dev(d["Ck"], dev))
    vb = kvc.BaseParams(centroids=to_dev(d["Cv"], dev))
    print(f"paired encode bits={bits} group={group} C={C} rot={rot}", flush=True)
    gk, gv = _pair_vs_single(codec, d, dev, kb, vb, 7, 300, 320)
    for g, name, cname in ((gk, "K", "Ck"), (gv, "V", "Cv")):
        check_centroid_store(g, nm.bf16_to_f32(d[name][:300]), nm.bf16_to_f32(d[cname]), bits, group,
                             rows=slice(7, 307), rotation=rot)
        assert np.all(g["codes"][:, :7] == 0xFFFFFFFF) and np.all(g["codes"][:, 307:] == 0xFFFFFFFF)


def test_paired_encode_other_bases_fall_back_to_two_launches():
    """A plain INT4 codec and temporal keys (AR(2) over two reconstructed frames) go
    through the general encoders, one tensor after the other."""
    dev = device()
    d = synth.cfg1(seed=42, hist_frames=3, query_frames=1, tokens=100, heads=3, dim=128,
                   n_centroids=16)
    print("paired encode: plain and temporal-key codecs", flush=True)
    _pair_vs_single(kvc.Codec(3, 128, 4, 32, kvc.BASE_NONE), d, dev, None, None, 0, 200, 200)
    rng = np.random.default_rng(3)
    prev = [to_dev(synth.bf16_bits(rng.standard_normal((200, 3, 128))), dev) for _ in range(2)]
    a = torch.from_numpy(rng.uniform(0.5, 1.0, (3, 128)).astype(np.float32)).to(dev)
    b = torch.from_numpy(rng.uniform(-0.2, 0.2, (3, 128)).astype(np.float32)).to(dev)
    base = kvc.BaseParams(prev0=prev[0], prev1=prev[1], coef_a=a, coef_b=b)
    _pair_vs_single(kvc.Codec(3, 128, 2, 32, kvc.BASE_TEMPORAL), d, dev, base, base, 0, 200, 200)


def test_paired_encode_cfg1_chunk_full_size():
    """The timed chunk of the default workload: 4680 tokens x 12 heads, 256 centroids,
    INT2 g32, written at row 28080 of the 32760-row history stores."""
    dev = device()
    d = synth.cfg1()
    lo, hi = d["chunk"]
    codec = kvc.Codec(12, 128, 2, 32, kvc.BASE_CENTROID, 256)
    kb = kvc.BaseParams(centroids=to_dev(d["Ck"], dev))
    vb = kvc.BaseParams(centroids=to_dev(d["Cv"], dev))
    K = to_dev(np.ascontiguousarray(d["K"][lo:hi]), dev)
    V = to_dev(np.ascontiguousarray(d["V"][lo:hi]), dev)
    n = d["K"].shape[0]
    pk, pv, sk, sv = (kvc.Store.allocate(codec, n, dev) for _ in range(4))
    print("paired encode of the cfg1 chunk", flush=True)
    kvc.kvc_encode_kv(codec, K, V, pk, pv, lo, kb, vb)
    kvc.kvc_encode(codec, K, sk, lo, kb)
    kvc.kvc_encode(codec, V, sv, lo, vb)
    torch.cuda.synchronize()
    for a, b in ((pk, sk), (pv, sv)):
        ga, gb = store_np(a), store_np(b)
        for key in ga:
            assert np.array_equal(ga[key][:, lo:hi], gb[key][:, lo:hi]), key


# every code width, group and rotation of the 16-token-wave encoder (rotations divide the group)
TWO_ROUND = [(b, g, r) for b in (2, 4) for g in (16, 32, 64) for r in (0, 16)] + [(2, 64, 64), (4, 64, 64)]


@pytest.mark.parametrize("bits,group,rot", TWO_ROUND)
def test_paired_encode_two_round_grid(bits, group, rot):
    """12 heads x 3000 tokens, 256 centroids: the paired launch's workgroups walk two tiles
    each, the single-tensor calls' one; both give the same stores, which match the oracle
    on the first 96 rows and the ragged last 40."""
    dev = device()
    d = synth.cfg1(seed=44, hist_frames=2, query_frames=1, tokens=1500, heads=12, dim=128,
                   n_centroids=256)
    codec = kvc.Codec(12, 128, bits, group, kvc.BASE_CENTROID, 256, rotation=rot)
    kb = kvc.BaseParams(centroids=to_dev(d["Ck"], dev))
    vb = kvc.BaseParams(centroids=to_dev(d["Cv"], dev))
    print(f"paired encode, two-round grid: bits={bits} group={group} rot={rot}", flush=True)
    gk, gv = _pair_vs_single(codec, d, dev, kb, vb, 0, 3000, 3000)
    for g, name, cname in ((gk, "K", "Ck"), (gv, "V", "Cv")):
        for r0, r1 in ((0, 96), (2960, 3000)):
            check_centroid_store(g, nm.bf16_to_f32(d[name][r0:r1]), nm.bf16_to_f32(d[cname]), bits,
                                 group, rows=slice(r0, r1), rotation=rot)
