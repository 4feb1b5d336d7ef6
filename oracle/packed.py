"""Oracle of the packed candidate-site buffer -- TEST INFRASTRUCTURE ONLY (only the
tests, the package smoke check and the benchmark's CPU baseline use it; the
product path never imports it).

Pages: paperlayer.ai summary, Appendix B.2 "Packed candidate sites": the
candidate-update kernels read a 16-byte per-site buffer of float16 pairs --
position, (log tau, r), anisotropy direction and (a, 0) -- regenerated after
densification to save bandwidth.

Readings (the pages give the fields, nothing more):
  * word order and halves: word 0 = (x, y), word 1 = (log tau, r), word 2 =
    (dir_x, dir_y), word 3 = (a, 0); the first field of a pair in the low 16 bits;
  * units: those of the site buffer (pixels for x, y, r);
  * rounding: IEEE 754 binary16, round to nearest even, overflow to infinity
    (numpy's float32 -> float16 conversion implements exactly this);
  * an inactive slot (x < 0 in float32) is packed with x = -1 (a tiny negative x
    would otherwise round to -0 and look active);
  * selection from the packed buffer is selection on the sites whose seven packed
    fields are replaced by their float16 values: the same score, ranking and
    filters, evaluated in float32 from the rounded parameters.  Colours are not
    packed (selection does not read them).
"""
import numpy as np

X, Y, LOGTAU, R, CR, CG, CB, DX, DY, A = range(10)
PACKED = (X, Y, LOGTAU, R, DX, DY, A)


def _halves(S, n):
    S = np.asarray(S, dtype=np.float32)[:, :n]
    with np.errstate(over="ignore"):  # overflow to infinity is the defined result
        h = {f: S[f].astype(np.float16) for f in PACKED}
    h[X] = np.where(S[X] < 0, np.float16(-1.0), h[X])
    return h


def pack_words(sites, n_slots) -> np.ndarray:
    """uint32 [n_slots][4]: the packed buffer's words."""
    h = _halves(sites, n_slots)
    b = {f: h[f].view(np.uint16).astype(np.uint32) for f in PACKED}
    out = np.empty((n_slots, 4), dtype=np.uint32)
    out[:, 0] = b[X] | (b[Y] << 16)
    out[:, 1] = b[LOGTAU] | (b[R] << 16)
    out[:, 2] = b[DX] | (b[DY] << 16)
    out[:, 3] = b[A]
    return out


def rounded_sites(sites, n_slots) -> np.ndarray:
    """The float32 site buffer that packed-mode selection sees: the seven packed
    fields of slots [0, n_slots) replaced by their float16 values (inactive x -> -1);
    colours and slots >= n_slots unchanged."""
    S = np.array(sites, dtype=np.float32, copy=True)
    h = _halves(S, n_slots)
    for f in PACKED:
        S[f, :n_slots] = h[f].astype(np.float32)
    return S
