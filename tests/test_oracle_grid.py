"""Pins of the oracle's downscaled candidate grid (paperlayer.ai summary,
Appendix B.3 "Candidate field": a ceil(W/c) x ceil(H/c) grid, pixels mapped to
cells by integer division, candidates evaluated at the centred cell UVs).

* the map has ceil(W/c) x ceil(H/c) entries, also for ragged sizes;
* for Euclidean sites (a = 0, r = 0) a cell's exact list is the 8 nearest sites of
  a k-d tree queried at ((cx + 1/2) W/Wm, (cy + 1/2) H/Hm) -- the centred UV in
  pixel units -- and not those of the cell's corner or of its first pixel;
* the render, its backward and the budget statistics with cell c equal the
  per-pixel versions on the map expanded to pixels by the integer mapping;
* for sizes divisible by a power-of-two c, selection on the grid (exact top-8,
  propagation with injection, the jump-flood seed and flood passes) is
  bit-identical to per-pixel selection on a W/c x H/c image whose sites' positions
  and radii are divided by c: every score is the same float32 number.
"""
import numpy as np
import pytest

import oracle
import synth

NONE = 0xFFFFFFFF


def _expand(m, W, H, c):
    """Per-pixel map from a cell map by the integer mapping (col // c, row // c)."""
    rows = np.arange(H) // c
    cols = np.arange(W) // c
    return np.ascontiguousarray(m[rows][:, cols])


def _scaled(S, n, c):
    T = S.copy()
    T[synth.X, :n] /= c
    T[synth.Y, :n] /= c
    T[synth.R, :n] /= c
    return T


@pytest.mark.parametrize("W,H,c", [(37, 23, 4), (64, 48, 2), (50, 31, 3), (5, 3, 8), (17, 1, 4)])
def test_grid_shape(orc, W, H, c):
    S = synth.random_sites(30, W, H, 5)
    m = orc.topk_exact(S, 30, W, H, cell=c)
    assert m.shape == (-(-H // c), -(-W // c), 8) == oracle.map_shape(W, H, c)
    assert orc.jfa_seed(S, 30, W, H, cell=c).shape == m.shape


@pytest.mark.parametrize("W,H,c", [(96, 64, 4), (101, 67, 4), (90, 50, 3), (64, 64, 8)])
def test_grid_euclidean_knn_at_cell_centres(orc, W, H, c):
    from scipy.spatial import cKDTree

    n = 500
    S = synth.random_sites(n, W, H, 51)
    S[synth.A] = 0.0
    S[synth.R] = 0.0
    m = orc.topk_exact(S, n, W, H, cell=c)
    Hm, Wm = m.shape[:2]
    cy, cx = np.divmod(np.arange(Wm * Hm), Wm)
    q = np.stack([(cx + 0.5) * (W / Wm), (cy + 0.5) * (H / Hm)], -1)
    tree = cKDTree(np.stack([S[synth.X, :n], S[synth.Y, :n]], -1).astype(np.float64))
    dist, idx = tree.query(q, k=9)
    got = m.reshape(-1, 8)
    ties = dist[:, 8] - dist[:, 7] < 1e-4
    same = np.array([set(a) == set(b) for a, b in zip(got, idx[:, :8])])
    assert (same | ties).all()
    assert same.mean() > 0.95
    # the centred UV matters: the lists at the cells' first pixels differ
    corner = np.stack([cx * c + 0.5, cy * c + 0.5], -1)
    _, idx0 = tree.query(corner, k=8)
    assert np.mean([set(a) == set(b) for a, b in zip(got, idx0)]) < 0.5


@pytest.mark.parametrize("W,H,c", [(37, 23, 4), (40, 24, 2), (33, 20, 3)])
def test_grid_render_equals_expanded_map(orc, W, H, c):
    n = 120
    S = synth.random_sites(n, W, H, 52, n + 4)
    S[synth.X, 7] = -1.0
    Wm, Hm = -(-W // c), -(-H // c)
    m = synth.random_map(Wm, Hm, n + 4, seed=53)
    tgt = (synth.pixel_noise(W, H, 54, 0.2) + 0.5).astype(np.float32)
    e = _expand(m, W, H, c)
    S64 = S.astype(np.float64)
    assert np.array_equal(orc.render_fwd(S64, n, m, W, H, cell=c), orc.render_fwd(S64, n, e, W, H))
    pix = np.array([0, W - 1, W * H - 1, (H // 2) * W + W // 3], dtype=np.uint32)
    assert np.array_equal(orc.render_fwd_pixels(S64, n, m, W, H, pix, cell=c),
                          orc.render_fwd_pixels(S64, n, e, W, H, pix))
    g1, l1 = orc.render_bwd(S64, n, m, tgt, W, H, cell=c)
    g2, l2 = orc.render_bwd(S64, n, e, tgt, W, H)
    assert np.array_equal(g1, g2) and l1 == l2
    assert np.array_equal(orc.densify_stats(S64, n, m, tgt, W, H, cell=c), orc.densify_stats(S64, n, e, tgt, W, H))


@pytest.mark.parametrize("W,H,c", [(64, 48, 4), (40, 24, 2), (96, 32, 8)])
def test_grid_selection_equals_scaled_image(orc, W, H, c):
    n = 300
    S = synth.random_sites(n, W, H, 55)
    S[synth.X, 4] = -1.0
    S[synth.X, 9] = float(W) + 3.0  # beyond the right border: seeds into the last column
    T = _scaled(S, n, c)
    Wm, Hm = W // c, H // c
    assert np.array_equal(orc.topk_exact(S, n, W, H, cell=c), orc.topk_exact(T, n, Wm, Hm))
    cin = synth.random_map(Wm, Hm, n + 2, seed=56)
    for jump, t in ((1, 0), (4, 3), (16, 7)):
        a = orc.propagate(S, n, cin, W, H, jump, t, synth.SEED_INJECT, 4, cell=c)
        b = orc.propagate(T, n, cin, Wm, Hm, jump, t, synth.SEED_INJECT, 4)
        assert np.array_equal(a, b)
    seed_c = orc.jfa_seed(S, n, W, H, cell=c)
    assert np.array_equal(seed_c, orc.jfa_seed(T, n, Wm, Hm))
    assert 9 in seed_c[:, -1]
    for k in orc.jfa_steps(W, H, cell=c):
        assert np.array_equal(orc.jfa_pass(S, n, cin, W, H, k, cell=c), orc.jfa_pass(T, n, cin, Wm, Hm, k))
    pix = np.arange(Wm * Hm, dtype=np.uint32)[::7]
    assert np.array_equal(orc.score_pairs(S, n, W, H, pix, pix % n, cell=c), orc.score_pairs(T, n, Wm, Hm, pix, pix % n))


def test_grid_schedules_count_map_entries():
    assert oracle.jump_schedule(768, 512, 12, cell=4) == [128, 64, 32, 16, 8, 4, 2, 1, 1, 1, 1, 1]
    assert oracle.jfa_steps(768, 512, cell=4) == [128, 64, 32, 16, 8, 4, 2, 1]
    assert oracle.jfa_steps(4, 4, cell=4) == []
