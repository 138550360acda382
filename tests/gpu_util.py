"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and
reading compressed stores back (data plumbing only, no codec arithmetic)."""
import numpy as np
import pytest
import torch

from oracle import codec as ocodec


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    """float32 arrays as fp32 tensors; uint16 arrays (bf16 bits) as bfloat16 tensors."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def store_np(st) -> dict:
    torch.cuda.synchronize()
    out = dict(codes=st.codes.cpu().numpy().view(np.uint32),
               scale_zero=st.scale_zero.cpu().numpy().view(np.uint32), index=None)
    if st.index is not None:
        idx = st.index.cpu().numpy()
        out["index"] = idx.view(np.uint16) if idx.dtype == np.int16 else idx
    return out


def fill_sentinel(st):
    """Pre-fill a store with a pattern the codec cannot produce everywhere at once."""
    st.codes.fill_(-1)
    st.scale_zero.fill_(-1)
    if st.index is not None:
        st.index.fill_(-1)


def bf16_to_f32_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def check_centroid_store(got: dict, x: np.ndarray, C: np.ndarray, bits: int, group: int,
                         rows=slice(None), window: float = 1e-5, rotation: int = 0):
    """Bit-exact comparison of a centroid-codec store against the oracle on token rows
    `rows` (head-major store).  Assignments may differ only inside the near-tie window
    (relative top-2 gap < `window`); for such tokens the GPU's index must itself lie in
    the window and the codes must equal the oracle quantizer run with the GPU's index."""
    want = ocodec.encode_centroid(x, C, bits, group, rotation=rotation)
    gi = got["index"][:, rows].T.astype(np.int64)           # [N, H]
    wi = want["idx"]
    diff = gi != wi
    n_tie = int(diff.sum())
    if n_tie:
        gap = ocodec.tie_gap(want["dist"])
        assert np.all(gap[diff] < window), "assignment differs outside the near-tie window"
        dist = want["dist"].astype(np.float64)
        d1 = dist.min(-1)
        dg = np.take_along_axis(dist, gi[..., None], -1)[..., 0]
        assert np.all((dg - d1)[diff] <= window * d1[diff])
        base = C[np.arange(C.shape[0])[None, :], gi]
        re = ocodec.encode_residual(x, base, bits, group, rotation)
        want_store = ocodec.to_store(re["q"], re["s16"], re["z16"], bits, gi, C.shape[1])
    else:
        want_store = want["store"]
    assert np.array_equal(got["codes"][:, rows], want_store["codes"]), "codes differ"
    assert np.array_equal(got["scale_zero"][:, rows], want_store["scale_zero"]), "scale/zero differ"
    return want, n_tie
