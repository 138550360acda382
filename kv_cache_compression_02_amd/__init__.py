"""Compressed KV-cache codec and attention for AMD MI355X (gfx950).

The compute path is libkvc.so (hand-written HIP kernels behind the C ABI in
include/kvc.h); ``kvc`` is a thin ctypes binding that marshals torch tensors
(device memory and the current stream) into it.
"""
from .kvc import (  # noqa: F401
    ATTEND_JENSEN, BASE_CENTROID, BASE_COEFF, BASE_DPLR, BASE_NONE, BASE_TEMPORAL, BF16, F32,
    BaseParams,
    Codec, KvcError, Store, kvc_attend_compressed, kvc_attend_compressed_chunk,
    kvc_attend_mixed_dim, kvc_centroid_tables, kvc_decode, kvc_fit_centroids,
    kvc_encode, kvc_encode_kv, kvc_encode_noalloc, kvc_store_bytes, kvc_workspace_bytes, lib,
)
