"""Seeded synthetic inputs for the Soft Anisotropic Diagrams (SAD) hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no score, no blend, no gradient).  Both the CPU oracle
tests and the GPU path take their inputs from here.

Site layout (pages: paperlayer.ai summary, Appendix B.2 "Site buffer"; the field
order follows the press article's section 5 list): ten float32 planes of
``stride`` entries each, in the order

    0 x   1 y   2 log_tau   3 r   4 R   5 G   6 B   7 dir_x   8 dir_y   9 a

Positions and radii are in pixels.  Slots at or beyond ``n`` are inactive
(x = y = -1), the marker the pages give for pruned sites.

Site generator "G1" (our recipe; the pages' datasets are not available):
p ~ U[0,W) x U[0,H), colour ~ U[0,1]^3, r ~ U[0,2] px, a ~ N(0, 0.5),
theta ~ U[0, pi), dir = (cos theta, sin theta), log_tau ~ U[2, 5].
"""
from __future__ import annotations

import dataclasses

import numpy as np

NPARAM = 10
X, Y, LOGTAU, R, CR, CG, CB, DX, DY, A = range(NPARAM)

SEED_MODEL = 1
SEED_TARGET_SITES = 2
SEED_NOISE = 3
SEED_INJECT = 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    W: int
    H: int
    n_sites: int
    capacity: int
    iters: int
    n_inject: int

    @property
    def P(self) -> int:
        return self.W * self.H


# The five workloads: a tiny case, a Kodak-shaped one, a 2k one, a DIV2K-shaped
# one with budget control, and a 4k edit-stress refresh.
WORKLOADS = {
    "tiny64": Workload("tiny64", 64, 64, 256, 256, 1, 4),
    "kodak768": Workload("kodak768", 768, 512, 50_000, 50_000, 200, 4),
    "img2048": Workload("img2048", 2048, 2048, 131_072, 131_072, 500, 4),
    "div2k2040": Workload("div2k2040", 2040, 1356, 200_000, 220_000, 300, 4),
    "edit4096": Workload("edit4096", 4096, 4096, 1_000_000, 1_000_000, 1, 8),
}


def empty_sites(capacity: int) -> np.ndarray:
    s = np.zeros((NPARAM, capacity), dtype=np.float32)
    s[X] = -1.0
    s[Y] = -1.0
    return s


def random_sites(n: int, W: int, H: int, seed: int, capacity: int | None = None) -> np.ndarray:
    """G1 sites, float32 SoA [10][capacity]; slots >= n inactive."""
    cap = n if capacity is None else capacity
    assert cap >= n
    rng = np.random.Generator(np.random.PCG64(seed))
    s = empty_sites(cap)
    s[X, :n] = rng.uniform(0.0, W, n)
    s[Y, :n] = rng.uniform(0.0, H, n)
    s[LOGTAU, :n] = rng.uniform(2.0, 5.0, n)
    s[R, :n] = rng.uniform(0.0, 2.0, n)
    s[CR:CB + 1, :n] = rng.uniform(0.0, 1.0, (3, n))
    theta = rng.uniform(0.0, np.pi, n)
    s[DX, :n] = np.cos(theta)
    s[DY, :n] = np.sin(theta)
    s[A, :n] = rng.normal(0.0, 0.5, n)
    # float32 positions drawn in [0, W) can round up to W; keep them inside.
    s[X, :n] = np.minimum(s[X, :n], np.nextafter(np.float32(W), np.float32(0)))
    s[Y, :n] = np.minimum(s[Y, :n], np.nextafter(np.float32(H), np.float32(0)))
    return s


def pixel_noise(W: int, H: int, seed: int = SEED_NOISE, sigma: float = 0.01) -> np.ndarray:
    """Per-channel N(0, sigma) noise, float32 [H][W][3]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.normal(0.0, sigma, (H, W, 3)).astype(np.float32)


def empty_map(W: int, H: int) -> np.ndarray:
    """All-sentinel candidate map, uint32 [H][W][8]."""
    return np.full((H, W, 8), 0xFFFFFFFF, dtype=np.uint32)


def random_map(W: int, H: int, n_slots: int, seed: int, p_invalid: float = 0.1,
               p_dup: float = 0.1) -> np.ndarray:
    """A random (not score-sorted) candidate map with sentinels and duplicate IDs.

    Used to exercise propagation and rendering on arbitrary lists.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    m = rng.integers(0, n_slots, (H, W, 8), dtype=np.uint64).astype(np.uint32)
    dup = rng.random((H, W, 8)) < p_dup
    src = rng.integers(0, 8, (H, W, 8))
    m = np.where(dup, np.take_along_axis(m, src, axis=2), m)
    inv = rng.random((H, W, 8)) < p_invalid
    m[inv] = 0xFFFFFFFF
    return m.astype(np.uint32)


def local_map(sites: np.ndarray, n: int, W: int, H: int, seed: int, radius: float = 12.0) -> np.ndarray:
    """A map whose lists hold random sites from a nearby grid bucket.

    Cheap way to get a spatially coherent (but not exact) map at any size without
    computing any score: each pixel draws 8 IDs among sites whose position falls
    within +-radius px (square window), else random IDs.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    cell = max(1, int(radius))
    gx = max(1, (W + cell - 1) // cell)
    gy = max(1, (H + cell - 1) // cell)
    px = sites[X, :n]
    py = sites[Y, :n]
    cx = np.clip((px // cell).astype(np.int64), 0, gx - 1)
    cy = np.clip((py // cell).astype(np.int64), 0, gy - 1)
    key = cy * gx + cx
    order = np.argsort(key, kind="stable")
    counts = np.bincount(key, minlength=gx * gy)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rows = np.arange(H)[:, None]
    cols = np.arange(W)[None, :]
    out = np.empty((H, W, 8), dtype=np.uint32)
    for j in range(8):
        ox = rng.integers(-1, 2, (H, W))
        oy = rng.integers(-1, 2, (H, W))
        bx = np.clip(cols // cell + ox, 0, gx - 1)
        by = np.clip(rows // cell + oy, 0, gy - 1)
        b = by * gx + bx
        c = counts[b]
        pick = (rng.random((H, W)) * np.maximum(c, 1)).astype(np.int64)
        idx = np.where(c > 0, order[np.minimum(starts[b] + pick, n - 1)],
                       rng.integers(0, n, (H, W)))
        out[:, :, j] = idx.astype(np.uint32)
    return out


# ---------------------------------------------------------------- img2048 target
def polygon_image(W: int, H: int, seed: int, n_poly: int = 64, n_waves: int = 32) -> np.ndarray:
    """Seeded synthetic photo-like image, float32 [H][W][3] in [0,1].

    Mid-grey 0.5, plus n_poly convex polygons (hull of 3-8 uniform points) each
    adding a colour offset in U[-0.25, 0.25]^3, plus n_waves plane waves with
    wavelengths 16-128 px and amplitude 0.02; clamped to [0, 1].
    """
    from scipy.spatial import ConvexHull

    rng = np.random.Generator(np.random.PCG64(seed))
    img = np.full((H, W, 3), 0.5, dtype=np.float64)
    yy, xx = np.mgrid[0:H, 0:W]
    xc = xx + 0.5
    yc = yy + 0.5
    for _ in range(n_poly):
        k = int(rng.integers(3, 9))
        pts = np.stack([rng.uniform(0, W, k), rng.uniform(0, H, k)], axis=1)
        off = rng.uniform(-0.25, 0.25, 3)
        try:
            hull = ConvexHull(pts)
        except Exception:
            continue
        v = pts[hull.vertices]  # counter-clockwise
        x0, y0 = np.floor(v.min(0)).astype(int)
        x1, y1 = np.ceil(v.max(0)).astype(int)
        x0, y0 = max(x0, 0), max(y0, 0)
        x1, y1 = min(x1, W), min(y1, H)
        if x1 <= x0 or y1 <= y0:
            continue
        sx = xc[y0:y1, x0:x1]
        sy = yc[y0:y1, x0:x1]
        inside = np.ones(sx.shape, dtype=bool)
        for i in range(len(v)):
            ax, ay = v[i]
            bx, by = v[(i + 1) % len(v)]
            inside &= (bx - ax) * (sy - ay) - (by - ay) * (sx - ax) >= 0
        img[y0:y1, x0:x1][inside] += off
    for _ in range(n_waves):
        lam = rng.uniform(16, 128)
        ang = rng.uniform(0, 2 * np.pi)
        ph = rng.uniform(0, 2 * np.pi)
        col = rng.uniform(-1, 1, 3)
        w = np.sin(2 * np.pi / lam * (np.cos(ang) * xc + np.sin(ang) * yc) + ph)
        img += 0.02 * w[..., None] * col[None, None, :]
    return np.clip(img, 0.0, 1.0).astype(np.float32)


def gradient_weighted_sites(img: np.ndarray, n: int, seed: int, capacity: int | None = None,
                            mix: float = 0.7) -> np.ndarray:
    """Sites placed with density 0.7*|Sobel(lum)|/sum + 0.3/P; colour = image at the sample.

    Gradient-weighted initialization with a uniform prior (pages: paperlayer.ai
    summary, section 4 "Optimization"; the 0.7/0.3 mix is ours).
    Other fields as in G1.
    """
    H, W, _ = img.shape
    cap = n if capacity is None else capacity
    rng = np.random.Generator(np.random.PCG64(seed))
    lum = img @ np.array([0.299, 0.587, 0.114], dtype=np.float32)
    p = np.pad(lum, 1, mode="edge")
    gx = (p[:-2, 2:] + 2 * p[1:-1, 2:] + p[2:, 2:]) - (p[:-2, :-2] + 2 * p[1:-1, :-2] + p[2:, :-2])
    gy = (p[2:, :-2] + 2 * p[2:, 1:-1] + p[2:, 2:]) - (p[:-2, :-2] + 2 * p[:-2, 1:-1] + p[:-2, 2:])
    g = np.sqrt(gx.astype(np.float64) ** 2 + gy.astype(np.float64) ** 2).ravel()
    P = W * H
    tot = g.sum()
    dens = (mix * g / tot if tot > 0 else 0.0) + (1.0 - mix) / P
    dens = dens / dens.sum()
    pix = rng.choice(P, size=n, replace=True, p=dens)
    s = random_sites(n, W, H, seed + 1000, cap)
    s[X, :n] = (pix % W) + rng.uniform(0, 1, n)
    s[Y, :n] = (pix // W) + rng.uniform(0, 1, n)
    s[X, :n] = np.minimum(s[X, :n], np.nextafter(np.float32(W), np.float32(0)))
    s[Y, :n] = np.minimum(s[Y, :n], np.nextafter(np.float32(H), np.float32(0)))
    flat = img.reshape(-1, 3)
    s[CR:CB + 1, :n] = flat[pix].T
    return s


def displace_sites(sites: np.ndarray, n: int, W: int, H: int, seed: int, frac: float = 0.1,
                   amp: float = 256.0) -> np.ndarray:
    """Edit stress: move a seeded fraction of sites by U[-amp, amp]^2 px, clamped into the image."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = sites.copy()
    k = int(round(frac * n))
    idx = rng.choice(n, size=k, replace=False)
    s[X, idx] = np.clip(s[X, idx] + rng.uniform(-amp, amp, k), 0.0, np.float32(W) - 1e-3)
    s[Y, idx] = np.clip(s[Y, idx] + rng.uniform(-amp, amp, k), 0.0, np.float32(H) - 1e-3)
    return s
