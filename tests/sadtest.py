"""Shared helpers of the parity tests: moving arrays to the GPU and comparing
GPU results with the oracle under the tolerances the method's statement fixes:
candidate sets identical except where scores differ by < 1e-6, forward colours
within 1e-5 max abs, gradients within 1e-4 relative L2 per plane."""
import numpy as np
import torch

NONE = 0xFFFFFFFF
SCORE_TOL = 1e-6
FWD_TOL = 1e-5
GRAD_TOL = 1e-4


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def map_to_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def compare_lists(orc, S, n, W, H, pix, gpu_lists, ref_lists, unions=None, counts=None, cell=1):
    """Compare per-pixel candidate lists.  Returns the number of pixels whose sets
    differ; every such pixel must differ only by near-ties: after re-scoring both
    lists with the oracle (float32 selection score), the sorted scores agree within
    SCORE_TOL, the GPU list holds distinct usable IDs from the candidate union, and
    the sentinel pads the tail.  GPU lists must also be stored in ascending score
    order up to near-ties.  `pix` indexes map entries (cells of `cell` x `cell`
    pixels; single pixels when cell is 1)."""
    gpu_lists = np.asarray(gpu_lists).reshape(-1, 8)
    ref_lists = np.asarray(ref_lists).reshape(-1, 8)
    pix = np.asarray(pix, dtype=np.uint32).ravel()
    # sentinel padding and ordering of every GPU list
    valid = gpu_lists != NONE
    nval = valid.sum(1)
    assert (valid == (np.arange(8)[None, :] < nval[:, None])).all(), "GPU lists must be sentinel-padded at the tail"
    sc = orc.score_pairs(S, n, W, H, np.repeat(pix, 8), gpu_lists.ravel(), cell).reshape(-1, 8)
    assert np.isfinite(sc[valid]).all(), "GPU list holds an unusable ID"
    sc_m = np.where(valid, sc, np.inf)
    dif = np.diff(sc_m, axis=1)
    ok_order = (dif >= -SCORE_TOL) | ~np.isfinite(dif)
    assert ok_order.all(), "GPU list not in ascending score order"
    mism = np.array([set(a) != set(b) for a, b in zip(gpu_lists, ref_lists)])
    idx = np.nonzero(mism)[0]
    if idx.size:
        rsc = orc.score_pairs(S, n, W, H, np.repeat(pix[idx], 8), ref_lists[idx].ravel(), cell).reshape(-1, 8)
        for j, i in enumerate(idx):
            g = gpu_lists[i][gpu_lists[i] != NONE]
            assert len(set(g.tolist())) == g.size, f"duplicate IDs at pixel {pix[i]}"
            assert g.size == (ref_lists[i] != NONE).sum(), f"list length differs at pixel {pix[i]}"
            if unions is not None:
                assert set(g.tolist()) <= set(unions[i][:counts[i]].tolist()), f"ID outside the union at {pix[i]}"
            a = np.sort(sc[i][gpu_lists[i] != NONE])
            b = np.sort(rsc[j][ref_lists[i] != NONE])
            assert np.abs(a - b).max() <= SCORE_TOL, f"pixel {pix[i]}: scores {a} vs {b}"
    return int(idx.size)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)
