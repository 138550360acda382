"""Plain, slow CPU oracle of the predict-then-quantize KV codec and of attention
over the compressed history.

TEST INFRASTRUCTURE. Only the tests, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from this package;
the HIP library and its Python binding never do, and the two share no code.

What it follows (pages: NanoKV project page; NanoKV arXiv 2611.06377; Coral-KV
arXiv 2610.12514; TempoKV arXiv 2610.15324):

* ``codec``     nearest-centroid assignment, group-wise INTb residual quantizer,
                bit packing, decode (NanoKV abstract; Coral-KV abstract, Fig. 2c,
                Fig. 5c, Table 9 caption).
* ``rotation``  Hn residual transform: an orthonormal Sylvester-Hadamard rotation of
                each group of n residual channels before the quantizer (Coral-KV
                Fig. 5, Fig. 9b-c).
* ``fit``       online centroid fitting at block fill: Lloyd iterations whose
                assignment is the codec's nearest-centroid search (Coral-KV Fig. 2c).
* ``predict``   block-diagonal-plus-low-rank cross-layer predictors (Coral-KV
                Fig. 3) and temporal key / cross value predictors (TempoKV Fig. 2b).
* ``coeff``     coefficients of the centroid residual on a low-dimensional basis
                (NanoKV abstract: joint head-channel residuals as low-bit coefficients).
* ``attention`` dense softmax attention over the decoded cache and NanoKV-Fast
                style mixed-dimensional scoring (NanoKV abstract; "37.93% less
                historical-attention computation").
* ``ratio``     closed-form bits per element and compression ratio (TempoKV
                Tables 1-3, 7, 8; NanoKV "nominal 32x coefficient compression").

Numeric rules: the codec runs in IEEE binary32 with round-to-nearest-even on
every operation, no fused multiply-add, correctly rounded division, and
ascending-index order in every sum whose result decides an integer output.
Attention and the linear predictors are evaluated exactly in fp64.

Parity status: every function is pinned by the ``-m "not gpu"`` tests (brute
force, closed forms, special cases, library routines, the pages' printed
compression ratios); see the per-module docstrings.
"""
from . import numerics, rotation, codec, fit, predict, coeff, attention, ratio  # noqa: F401
