"""Pins for the closed-form compression ratio against the figures printed on the pages."""
import json
import os

import numpy as np

from conftest import GOLDEN
from oracle import ratio


def _g():
    with open(os.path.join(GOLDEN, "compression_ratios.json")) as f:
        return json.load(f)


def test_per_group_baselines():
    g = _g()
    for key, bits in (("int2_per_group_baseline", 2), ("int4_per_group_baseline", 4)):
        r = ratio.ratio(ratio.bits_per_element(bits, 32, 128))
        assert round(r, g[key]["printed_digits"]) == g[key]["ratio"]


def test_nanokv_nominal_coefficient_compression():
    g = _g()["nanokv_nominal_coefficient"]
    bpe = ratio.coeff_bits_per_element(16, 4, 128, sz=False)
    assert ratio.ratio(bpe) == g["ratio"]


def test_anchor_sweep_is_linear_in_anchor_bits():
    g = _g()["tempokv_anchor_sweep"]
    ab = np.array(g["anchor_bits"], dtype=float)
    bpe = 16.0 / np.array(g["ratio"])
    slope, icpt = np.polyfit(ab, bpe, 1)
    # printed to 3 decimals: each bits-per-element value is known to +-16*0.0005/ratio^2
    tol = 16 * 0.0005 / np.array(g["ratio"]) ** 2
    assert np.all(np.abs(icpt + slope * ab - bpe) <= tol)
    # the closed form's anchor term has exactly that slope: f per anchor bit
    f = slope
    ours = [ratio.bits_per_element(2, 64, 128, anchor_fraction=f, anchor_bits=int(b)) for b in ab]
    assert np.allclose(np.diff(ours), f, rtol=1e-12)
    assert 1 / 200 < f < 1 / 160   # about one anchor frame per ~180 frames


def test_config_bits_per_element():
    # centroid + INT2 g32 with uint8 index at d = 128: 2 + 1 + 8/128
    assert ratio.bits_per_element(2, 32, 128, index_bits=ratio.stored_index_bits(256)) == 3.0625
    assert ratio.information_index_bits(512) == 9 and ratio.stored_index_bits(512) == 16
    # coefficient keys, m = 16 INT4 with one fp16 scale/zero per token-head and uint16 index
    k = ratio.coeff_bits_per_element(16, 4, 128) + 16 / 128
    assert k == 0.5 + 0.25 + 0.125
