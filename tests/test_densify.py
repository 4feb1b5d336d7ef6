"""Budget control (densify / prune), CPU side.

* The oracle's per-site statistics are pinned to closed forms (one site covering
  the image) and to image-space identities (per-pixel weights sum to one, so the
  site sums of mass, energy and moments equal plain pixel sums).
* The oracle's split/prune rules are pinned to hand-built cases: a known
  covariance must split along its principal axis by half its standard deviation,
  a luminance ramp must split along its gradient, pruning takes the smallest
  removal deltas, children carry the target colour and fresh Adam state.
* The library's host routine sad_densify_prune is then compared with the oracle
  on seeded cases (statistics computed by the oracle, never by the GPU path).

Parity unpinned against the pages for the constants (fractions, alpha, shrink,
offset length): the pages do not state them.
"""
import math

import numpy as np
import pytest

import soft_voronoi_render_amd as sad
import synth
from oracle.densify import densify_prune as orc_densify

X, Y, LOGTAU, R, CR, CG, CB, DX, DY, A = range(10)
NONE = 0xFFFFFFFF


def _one_site_case(W, H, px, py, col, tgt):
    S = synth.empty_sites(1)
    S[:, 0] = [px, py, 3.0, 0.5, col[0], col[1], col[2], 0.6, 0.8, 0.3]
    cand = np.full((H, W, 8), NONE, dtype=np.uint32)
    cand[..., 0] = 0
    T = np.empty((H, W, 3), dtype=np.float32)
    T[...] = tgt
    return S, cand, T


@pytest.mark.parametrize("W,H,px,py", [(7, 5, 2.25, 3.5), (16, 9, 0.0, 9.0), (1, 3, 0.5, 1.0)])
def test_stats_one_site_closed_form(orc, W, H, px, py):
    col, tgt = (0.25, 0.5, 1.0), (0.75, 0.125, 0.5)
    S, cand, T = _one_site_case(W, H, px, py, col, tgt)
    st = orc.densify_stats(S, 1, cand, T, W, H)[0]
    e = sum((np.float64(np.float32(a)) - np.float64(np.float32(b))) ** 2 for a, b in zip(col, tgt))
    sx = W * W / 2 - W * px            # sum over columns of (col + 0.5 - px)
    sy = H * H / 2 - H * py
    sxx = (W ** 3 / 3 - W / 12) - px * W * W + W * px * px
    syy = (H ** 3 / 3 - H / 12) - py * H * H + H * py * py
    want = [W * H, e * W * H, e * H * sx, e * W * sy, e * H * sxx, e * sx * sy, e * W * syy, 0.0]
    assert np.allclose(st, want, rtol=1e-12, atol=1e-12)


def test_stats_pixel_sum_identities(orc):
    W, H, n = 40, 28, 120
    S = synth.random_sites(n, W, H, 11, n + 8)
    S[0, 5] = S[1, 5] = -1.0  # an inactive slot referenced by the lists
    cand = synth.random_map(W, H, n, seed=12)
    T = (synth.pixel_noise(W, H, 13, 0.3) + 0.5).astype(np.float32)
    st = orc.densify_stats(S, n, cand, T, W, H)
    img = orc.render_fwd(S, n, cand, W, H)
    e = ((img - T.astype(np.float64)) ** 2).sum(-1)
    # pixels whose list holds at least one active, finite site
    valid = (cand < n) & ~(S[0, np.minimum(cand, n - 1)] < 0)
    nonempty = valid.any(-1)
    assert st[:, 0].sum() == pytest.approx(nonempty.sum(), rel=1e-12)
    assert st[:, 1].sum() == pytest.approx(e.sum(), rel=1e-12)
    Xc = np.arange(W)[None, :] + 0.5 + np.zeros((H, 1))
    Yc = np.arange(H)[:, None] + 0.5 + np.zeros((1, W))
    px, py = S[0].astype(np.float64), S[1].astype(np.float64)
    E1 = st[:, 1]
    # first and second moments about the origin, summed over sites == pixel sums
    assert (st[:, 2] + E1 * px).sum() == pytest.approx((e * Xc).sum(), rel=1e-10)
    assert (st[:, 3] + E1 * py).sum() == pytest.approx((e * Yc).sum(), rel=1e-10)
    assert (st[:, 4] + 2 * px * st[:, 2] + px * px * E1).sum() == pytest.approx((e * Xc * Xc).sum(), rel=1e-10)
    assert (st[:, 6] + 2 * py * st[:, 3] + py * py * E1).sum() == pytest.approx((e * Yc * Yc).sum(), rel=1e-10)
    xy = st[:, 5] + py * st[:, 2] + px * st[:, 3] + px * py * E1
    assert xy.sum() == pytest.approx((e * Xc * Yc).sum(), rel=1e-10)
    assert np.all(st[n:] == 0)


def _budget_case(n=6, cap=10, W=32, H=24):
    S = synth.empty_sites(cap)
    rng = np.random.default_rng(5)
    for i in range(n):
        S[:, i] = [4 + 4 * i, 6 + 2 * i, 3.0 + 0.1 * i, 0.4 + 0.1 * i, 0.1, 0.2, 0.3, 1.0, 0.0, 0.2 * i]
    m = rng.random((10, cap)).astype(np.float32)
    v = rng.random((10, cap)).astype(np.float32)
    stats = np.zeros((cap, 8), dtype=np.float32)
    removal = np.zeros(cap, dtype=np.float32)
    cand = np.full((H, W, 8), NONE, dtype=np.uint32)
    T = np.zeros((H, W, 3), dtype=np.float32)
    return S, m, v, stats, removal, cand, T


def _cov_stats(E, lam1, lam2, theta, mass):
    c, s = math.cos(theta), math.sin(theta)
    C = np.array([[c, -s], [s, c]]) @ np.diag([lam1, lam2]) @ np.array([[c, s], [-s, c]])
    # zero mean offset: second moments about the site equal E * covariance
    return [mass, E, 0.0, 0.0, E * C[0, 0], E * C[0, 1], E * C[1, 1], 0.0]


@pytest.mark.parametrize("theta", [0.0, 0.4, math.pi / 2, 2.5])
def test_split_along_principal_axis(theta):
    S, m, v, stats, removal, cand, T = _budget_case()
    T[...] = (0.9, 0.5, 0.1)
    stats[2] = _cov_stats(3.0, 4.0, 1.0, theta, 50.0)
    for i in range(6):
        if i != 2:
            stats[i] = [50.0, 0.1, 0, 0, 0.1, 0, 0.1, 0]
    removal[:6] = [5, 6, 7, 8, 9, 10]
    parent = S[:, 2].copy()
    n, ns, npr, short = orc_densify(S, m, v, 6, 10, stats, removal, cand, 32, 24, T, split_frac=1 / 6,
                                    prune_frac=0.0)
    assert (n, ns, npr, short) == (7, 1, 0, False)
    a, b = S[:, 2], S[:, 6]
    ax = np.array([math.cos(theta), math.sin(theta)])
    if ax[0] < -1e-12 or (abs(ax[0]) <= 1e-12 and ax[1] < 0):
        ax = -ax
    half = 0.5 * math.sqrt(4.0)
    assert np.allclose(a[:2], parent[:2] - half * ax, atol=1e-5)
    assert np.allclose(b[:2], parent[:2] + half * ax, atol=1e-5)
    for c in (a, b):
        assert np.allclose(c[CR:CB + 1], (0.9, 0.5, 0.1))
        assert c[R] == np.float32(parent[R] * np.float32(0.85))
        assert c[LOGTAU] == pytest.approx(parent[LOGTAU] + math.log(0.85), abs=1e-6)
        assert np.array_equal(c[DX:], parent[DX:])
    assert np.all(m[:, [2, 6]] == 0) and np.all(v[:, [2, 6]] == 0)
    assert m[0, 1] != 0  # untouched sites keep their Adam state
    # child B is seeded into its pixel's list and the four neighbours'
    bc, br = int(b[X]), int(b[Y])
    for dc, dr in ((0, 0), (-1, 0), (1, 0), (0, -1), (0, 1)):
        assert cand[br + dr, bc + dc, 7] == 6
    assert (cand[..., 7] == 6).sum() == 5 and np.all(cand[..., :7] == NONE)


@pytest.mark.parametrize("cell", [2, 5])
def test_split_seeds_the_cell_map(cell):
    """On a map of cells, child B enters the list of the cell that holds its pixel
    and of the four neighbour cells (inside the map)."""
    W, H = 32, 24
    S, m, v, stats, removal, _, T = _budget_case()
    Hm, Wm = -(-H // cell), -(-W // cell)
    cand = np.full((Hm, Wm, 8), NONE, dtype=np.uint32)
    stats[2] = _cov_stats(3.0, 4.0, 1.0, 0.3, 50.0)
    for i in range(6):
        if i != 2:
            stats[i] = [50.0, 0.1, 0, 0, 0.1, 0, 0.1, 0]
    n, ns, _, _ = orc_densify(S, m, v, 6, 10, stats, removal, cand, W, H, T, split_frac=1 / 6, prune_frac=0.0,
                              cell=cell)
    assert (n, ns) == (7, 1)
    bc, br = int(S[X, 6]) // cell, int(S[Y, 6]) // cell
    want = {(br + dr, bc + dc) for dc, dr in ((0, 0), (-1, 0), (1, 0), (0, -1), (0, 1))
            if 0 <= br + dr < Hm and 0 <= bc + dc < Wm}
    assert {tuple(x) for x in np.argwhere(cand[..., 7] == 6)} == want
    assert np.all(cand[..., :7] == NONE)


@pytest.mark.parametrize("direction", ["x", "y", "flat"])
def test_split_low_mass_uses_sobel_axis(direction):
    S, m, v, stats, removal, cand, T = _budget_case()
    Hh, Ww = T.shape[:2]
    ramp = np.arange(Ww if direction == "x" else Hh, dtype=np.float32) / 64
    if direction == "x":
        T[...] = ramp[None, :, None]
    elif direction == "y":
        T[...] = ramp[:, None, None]
    else:
        T[...] = 0.5
    stats[3] = [0.5, 2.0, 0, 0, 1.0, 0, 1.0, 0]  # mass below min_mass -> gradient axis
    removal[:6] = 1.0
    parent = S[:, 3].copy()
    n, ns, npr, short = orc_densify(S, m, v, 6, 10, stats, removal, cand, 32, 24, T, split_frac=0.2,
                                    prune_frac=0.0)
    assert (ns, npr) == (1, 0)
    ax = {"x": (1.0, 0.0), "y": (0.0, 1.0), "flat": (1.0, 0.0)}[direction]
    half = 0.5 * math.sqrt(1.0 / math.pi)
    assert np.allclose(S[:2, 3], parent[:2] - half * np.array(ax), atol=1e-6)
    assert np.allclose(S[:2, 6], parent[:2] + half * np.array(ax), atol=1e-6)


def test_prune_smallest_removal_and_free_slot_reuse():
    S, m, v, stats, removal, cand, T = _budget_case(n=10, cap=10)
    for i in range(10):
        stats[i] = [20.0, 1.0 + i, 0, 0, 1.0, 0, 2.0, 0]   # site 9 has the largest score
    removal[:10] = [3, 1, 4, 1, 5, 9, 2, 6, 5, 3]
    S[X, 4] = S[Y, 4] = -1.0                            # already inactive: not counted, slot free
    n, ns, npr, short = orc_densify(S, m, v, 10, 10, stats, removal, cand, 32, 24, T, split_frac=0.2,
                                    prune_frac=0.25)
    # A = 9 active -> 1 split (site 9), 2 prunes (removal 1 at sites 1 and 3; ties by ID)
    assert (n, ns, npr, short) == (10, 1, 2, False)
    # free slots, ascending: 1 and 3 (just pruned), 4 (inactive before); child B takes slot 1
    assert S[X, 3] == -1 and S[Y, 3] == -1 and S[X, 4] == -1
    assert S[X, 1] >= 0 and (cand[..., 7] == 1).sum() >= 3
    assert np.all(m[:, [1, 3, 9]] == 0) and np.all(v[:, [1, 3, 9]] == 0)
    active = ~(S[X, :10] < 0)
    assert active.sum() == 9 - 2 + 1


def test_capacity_shortage_reports():
    S, m, v, stats, removal, cand, T = _budget_case(n=6, cap=7)
    for i in range(6):
        stats[i] = [10.0, 1.0 + i, 0, 0, 1.0, 0, 1.0, 0]
    n, ns, npr, short = orc_densify(S, m, v, 6, 7, stats, removal, cand, 32, 24, T, split_frac=0.5,
                                    prune_frac=0.0)
    assert (n, ns, npr, short) == (7, 1, 0, True)


def _random_budget_case(seed, W=48, H=40, n=300, cap=330, inactive=6, cell=1):
    import oracle
    S = synth.random_sites(n, W, H, seed, cap)
    rng = np.random.default_rng(seed)
    dead = rng.choice(n, inactive, replace=False)
    S[0, dead] = S[1, dead] = -1.0
    if cell == 1:
        cand = synth.local_map(S, n, W, H, seed=seed + 1, radius=6.0)
    else:
        cand = oracle.topk_exact(S, n, W, H, cell=cell)
    T = (synth.pixel_noise(W, H, seed + 2, 0.2) + 0.5).astype(np.float32)
    stats = oracle.densify_stats(S, n, cand, T, W, H, cell=cell).astype(np.float32)
    removal = rng.normal(0, 1, cap).astype(np.float32)
    removal[rng.choice(n, 4, replace=False)] = np.nan
    m = rng.normal(0, 1, (10, cap)).astype(np.float32)
    v = rng.random((10, cap)).astype(np.float32)
    return S, m, v, stats, removal, cand, T


@pytest.mark.parametrize("seed,cfg,cell", [
    (1, sad.BudgetConfig(), 1),
    (2, sad.BudgetConfig(split_frac=0.2, prune_frac=0.0), 1),             # runs out of slots
    (3, sad.BudgetConfig(split_frac=0.1, prune_frac=0.1, min_mass=1e6), 1),  # gradient axis throughout
    (4, sad.BudgetConfig(split_frac=0.08, prune_frac=0.02, alpha=0.0, shrink=0.7), 1),
    (5, sad.BudgetConfig(split_frac=0.0, prune_frac=0.3), 1),
    (6, sad.BudgetConfig(split_frac=0.1, prune_frac=0.05), 3),           # map of 3x3-pixel cells
    (7, sad.BudgetConfig(split_frac=0.2, prune_frac=0.1), 8),
])
def test_host_densify_matches_oracle(orc, seed, cfg, cell):
    W, H, n, cap = 48, 40, 300, 330
    case = _random_budget_case(seed, W, H, n, cap, cell=cell)
    mine = [a.copy() for a in case]
    ref = [a.copy() for a in case]
    got = sad.densify_prune_stats(mine[0], mine[1], mine[2], n, cap, mine[3], mine[4], mine[5], W, H, mine[6], cfg,
                            cell=cell)
    f32 = lambda x: float(np.float32(x))  # the C struct holds float32 constants
    want = orc_densify(ref[0], ref[1], ref[2], n, cap, ref[3], ref[4], ref[5], W, H, ref[6],
                       f32(cfg.split_frac), f32(cfg.prune_frac), f32(cfg.alpha), f32(cfg.min_mass), f32(cfg.shrink),
                       cell=cell)
    assert got[:3] == want[:3]
    assert (got[3] == sad.SAD_ERR_CAPACITY) == want[3]
    assert np.allclose(mine[0][:2], ref[0][:2], atol=2e-5)
    assert np.allclose(mine[0][2:], ref[0][2:], atol=1e-6, equal_nan=True)
    assert np.array_equal(mine[1], ref[1]) and np.array_equal(mine[2], ref[2])
    assert np.array_equal(mine[5], ref[5])
    assert got[1] > 0 or cfg.split_frac == 0


def test_host_densify_matches_oracle_at_threaded_sizes(orc):
    """Large enough that every phase of the routine runs on several host threads
    (scores of 20 000 sites, about 5000 splits and 5000 prunes): the result must
    still equal the oracle's, which takes the splits one by one in order."""
    W, H, n, cap = 256, 192, 20000, 21000
    case = _random_budget_case(8, W, H, n, cap, inactive=40)
    cfg = sad.BudgetConfig(split_frac=0.25, prune_frac=0.25)
    mine = [a.copy() for a in case]
    ref = [a.copy() for a in case]
    got = sad.densify_prune_stats(mine[0], mine[1], mine[2], n, cap, mine[3], mine[4], mine[5], W, H, mine[6], cfg)
    f32 = lambda x: float(np.float32(x))
    want = orc_densify(ref[0], ref[1], ref[2], n, cap, ref[3], ref[4], ref[5], W, H, ref[6],
                       f32(cfg.split_frac), f32(cfg.prune_frac), f32(cfg.alpha), f32(cfg.min_mass), f32(cfg.shrink))
    assert got[:3] == want[:3] and got[1] > 4096 and got[2] > 4096
    assert (got[3] == sad.SAD_ERR_CAPACITY) == want[3]
    assert np.allclose(mine[0][:2], ref[0][:2], atol=2e-5)
    assert np.allclose(mine[0][2:], ref[0][2:], atol=1e-6, equal_nan=True)
    assert np.array_equal(mine[1], ref[1]) and np.array_equal(mine[2], ref[2])
    assert np.array_equal(mine[5], ref[5])


def test_host_densify_rejects_bad_arguments():
    W, H, n, cap = 16, 12, 20, 24
    S, m, v, stats, removal, cand, T = _random_budget_case(7, W, H, n, cap, inactive=0)
    for bad in (sad.BudgetConfig(split_frac=-0.1), sad.BudgetConfig(prune_frac=1.5), sad.BudgetConfig(shrink=0.0),
                sad.BudgetConfig(min_mass=-1.0)):
        with pytest.raises(sad.SadError):
            sad.densify_prune_stats(S, m, v, n, cap, stats, removal, cand, W, H, T, bad)
    with pytest.raises(sad.SadError):
        sad.densify_prune_stats(S, m, v, n, n - 1, stats, removal, cand, W, H, T)  # capacity < n
    with pytest.raises(ValueError):
        sad.densify_prune_stats(S, m, v, n, cap, stats[:-1], removal, cand, W, H, T)
    with pytest.raises(TypeError):
        sad.densify_prune_stats(S.astype(np.float64), m, v, n, cap, stats, removal, cand, W, H, T)


@pytest.mark.parametrize("cell", [1, 3])
def test_host_densify_seed_pairs_reproduce_the_map(cell):
    """With the map left on the device, the routine reports the entries it seeds,
    grouped by entry; applying them in order with the seeding rule (the last place
    takes the ID unless the list already names it) gives exactly the map it writes
    when it is handed the map, and everything else is the same."""
    import oracle
    W, H, n, cap = 48, 40, 300, 330
    case = _random_budget_case(8, W, H, n, cap, cell=cell)
    cfg = sad.BudgetConfig(split_frac=0.2, prune_frac=0.05)
    a = [x.copy() for x in case]
    b = [x.copy() for x in case]
    ra = sad.densify_prune_stats(a[0], a[1], a[2], n, cap, a[3], a[4], a[5], W, H, a[6], cfg, cell=cell)
    rb = sad.densify_prune_stats(b[0], b[1], b[2], n, cap, b[3], b[4], None, W, H, b[6], cfg, cell=cell, want_seeds=True)
    assert ra == rb[:4] and ra[1] > 0
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    seeds = rb[4]
    assert seeds.shape[1] == 2 and 0 < len(seeds) <= 5 * ra[1]
    e = seeds[:, 0].astype(np.int64)
    assert (np.diff(e) >= 0).all(), "pairs grouped by entry"
    m = case[5].copy().reshape(-1, 8)
    for e, i in seeds:
        if not (m[e] == i).any():
            m[e, 7] = i
    assert np.array_equal(m.reshape(a[5].shape), a[5])


@pytest.mark.parametrize("cell", [1, 2])
def test_densify_keeps_lists_distinct(cell):
    """A second child that takes a slot pruned in the same call keeps that slot's
    ID; lists near the pruned site's old place still name it, and one of them can
    be among the lists the child is seeded into.  Seeding skips such a list, so
    every list keeps distinct IDs (library routine and oracle alike)."""
    import oracle.densify as od
    W, H, n, cap = 40, 32, 60, 60
    Wm, Hm = -(-W // cell), -(-H // cell)
    rng = np.random.default_rng(3)
    S = synth.random_sites(n, W, H, 11, cap)
    stats = np.zeros((cap, 8), dtype=np.float32)
    stats[:n, 0] = 4.0
    stats[:n, 1] = rng.uniform(0.1, 1.0, n)
    stats[5, 1] = 100.0   # site 5 splits first, along +x (isotropic stats: no covariance)
    removal = rng.uniform(1.0, 2.0, cap).astype(np.float32)
    removal[7] = 0.0      # site 7 is pruned first; the second child of site 5 takes its slot
    S[0, 5], S[1, 5] = 20.5, 16.5
    # every list near site 5 names site 7 (the stale ID of the slot child B takes)
    cand = np.full((Hm, Wm, 8), 0xFFFFFFFF, dtype=np.uint32)
    cand[:, :, 0] = 7
    cand[:, :, 1] = 5
    T = (synth.pixel_noise(W, H, 4, 0.2) + 0.5).astype(np.float32)
    cfg = dict(split_frac=1.5 / n, prune_frac=1.5 / n, alpha=0.5, min_mass=1.0, shrink=0.85)
    for impl in ("library", "oracle"):
        a = [x.copy() for x in (S, np.zeros((10, cap), np.float32), np.zeros((10, cap), np.float32), cand)]
        if impl == "library":
            res = sad.densify_prune_stats(a[0], a[1], a[2], n, cap, stats, removal, a[3], W, H, T,
                                          sad.BudgetConfig(**cfg), cell=cell)
            assert res[1] == 1 and res[2] == 1
        else:
            res = od.densify_prune(a[0], a[1], a[2], n, cap, stats, removal, a[3], W, H, T, cell=cell, **cfg)
            assert res[1] == 1 and res[2] == 1
        assert a[0][0, 7] >= 0, "slot 7 holds the second child"
        L = a[3].reshape(-1, 8)
        for lst in L:
            v = lst[lst != 0xFFFFFFFF]
            assert len(set(v.tolist())) == v.size, f"{impl}: duplicate IDs in a list"
        assert (L[:, 7] == 0xFFFFFFFF).all(), f"{impl}: every seeded list already named slot 7"


def test_host_densify_rejects_a_short_seed_buffer():
    import ctypes
    W, H, n, cap = 48, 40, 300, 330
    S, m, v, stats, removal, cand, T = _random_budget_case(9, W, H, n, cap)
    before = [x.copy() for x in (S, m, v)]
    c = sad.BudgetConfig(split_frac=0.2, prune_frac=0.05).to_c()
    ns, nsp, npr, nseed = ctypes.c_int(n), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_long(0)
    seeds = np.zeros((10, 2), dtype=np.uint32)  # 5 * floor(0.2 * A) pairs are needed
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rc = sad.lib().sad_densify_prune_stats(p(S), p(m), p(v), cap, cap, ctypes.byref(ns), p(stats), p(removal), None, W, H,
                                     1, p(T), ctypes.byref(c), ctypes.byref(nsp), ctypes.byref(npr), p(seeds),
                                     len(seeds), ctypes.byref(nseed))
    assert rc == sad.SAD_ERR_ARG and ns.value == n
    for x, y in zip((S, m, v), before):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("seed,cfg,W,H", [
    (21, sad.BudgetConfig(), 48, 40),
    (22, sad.BudgetConfig(split_frac=0.15, prune_frac=0.1), 61, 37),
    (23, sad.BudgetConfig(split_frac=0.1, prune_frac=0.05, min_mass=1e6), 40, 48),  # gradient axis throughout
    (24, sad.BudgetConfig(split_frac=0.2, prune_frac=0.0), 48, 40),                # runs out of slots
])
def test_site_buffer_densify_matches_the_oracle(orc, seed, cfg, W, H):
    """sad_densify_prune derives the statistics itself (on the host, in float64,
    over the per-pixel map) and resets the removal accumulator.  Reference: the
    oracle's statistics (rounded to float32, the width the rules read) through the
    oracle's rules.  The statistics only choose and place splits, so equal
    results pin both."""
    n, cap = 300, 330
    S, m, v, _, removal, cand, T = _random_budget_case(seed, W, H, n, cap)
    mine = [a.copy() for a in (S, m, v, removal, cand)]
    ref = [a.copy() for a in (S, m, v, removal, cand)]
    ns, rc = sad.densify_prune(mine[0], mine[1], mine[2], mine[3], n, cap, mine[4], W, H, T, cfg, seed=seed)
    stats = orc.densify_stats(S, n, cand, T, W, H).astype(np.float32)
    f32 = lambda x: float(np.float32(x))
    want = orc_densify(ref[0], ref[1], ref[2], n, cap, stats, ref[3], ref[4], W, H, T, f32(cfg.split_frac),
                       f32(cfg.prune_frac), f32(cfg.alpha), f32(cfg.min_mass), f32(cfg.shrink))
    assert ns == want[0]
    assert (rc == sad.SAD_ERR_CAPACITY) == want[3]
    assert np.allclose(mine[0][:2], ref[0][:2], atol=2e-5)
    assert np.allclose(mine[0][2:], ref[0][2:], atol=1e-6, equal_nan=True)
    assert np.array_equal(mine[1], ref[1]) and np.array_equal(mine[2], ref[2])
    assert np.array_equal(mine[4], ref[4])
    assert np.all(mine[3][:ns] == 0), "removal accumulator reset"
    assert want[1] > 0 or cfg.split_frac == 0
    # the seed is reserved: another seed gives the same result
    again = [a.copy() for a in (S, m, v, removal, cand)]
    sad.densify_prune(again[0], again[1], again[2], again[3], n, cap, again[4], W, H, T, cfg, seed=seed + 99)
    for x, y in zip(again, mine):
        assert np.array_equal(x, y, equal_nan=True)
