"""Synthetic inputs are deterministic, shaped as described, and subsettable."""
import numpy as np

import synth


def test_cfg0_shapes_and_determinism():
    a, b = synth.cfg0(), synth.cfg0()
    for key in ("K", "V", "Q", "Ck", "Cv"):
        assert np.array_equal(a[key], b[key])
    assert a["K"].shape == (256, 2, 64) and a["Q"].shape == (64, 2, 64)
    assert a["Ck"].shape == (2, 16, 64) and a["K"].dtype == np.float32


def test_small_video_config_shapes():
    d = synth.cfg1(hist_frames=2, query_frames=1, tokens=40, heads=2, dim=32, n_centroids=8)
    assert d["K"].shape == (80, 2, 32) and d["K"].dtype == np.uint16
    assert d["Q"].shape == (40, 2, 32) and d["Ck"].shape == (2, 8, 32)
    assert d["chunk"] == (0, 80)


def test_cfg2_chunks_reproduce_subsets():
    p = synth.cfg2_params(heads=2, dim=16, rank=4)
    full = list(synth.cfg2_layers(params=p, n_tokens=30, n_layers=3, chunk=10))
    sub = list(synth.cfg2_layers(params=p, n_tokens=30, n_layers=3, chunk=10, chunk_ids=[2]))
    for (kf, vf), (ks, vs) in zip(full, sub):
        assert np.array_equal(kf[20:30], ks) and np.array_equal(vf[20:30], vs)


def test_cfg3_small_shapes():
    d = synth.cfg3(n_frames=3, query_frames=1, tokens=10, heads=2, dim=16)
    assert d["K"].shape == (30, 2, 16) and d["V"].shape == (30, 2, 16) and d["Q"].shape == (10, 2, 16)
