"""Pins of the oracle's jump-flood prepass (paperlayer.ai summary, Appendix B.3
"Jump schedule": a seed pass, then ceil(log2 max(W, H)) flood passes over 3x3
neighbourhoods keeping the four closest sites).

* the seed pass equals its definition recomputed here (the <= 4 best sites by
  (d, ID) among those whose pixel contains them), including crowded pixels,
  inactive and non-finite sites and positions on or beyond the image border;
* a flood pass equals the brute-force top-4 of the union of the 3x3 lists' first
  four entries;
* with at most four sites every pixel ends with all of them, i.e. the exact top-4
  (orc.topk_exact, pinned against library KNN elsewhere);
* the exact top-4 is a fixed point of every flood pass;
* for Euclidean sites (a = 0, r = 0) the prepass finds a k-d tree's nearest site
  at nearly every pixel (jump flooding is approximate; the pages give no rate).
"""
import numpy as np
import pytest

import oracle
import synth

NONE = 0xFFFFFFFF


def _expected_seed(orc, S, n, W, H):
    x, y = S[synth.X, :n], S[synth.Y, :n]
    ok = ~(x < 0) & np.isfinite(x) & np.isfinite(y)
    col = np.floor(np.clip(np.nan_to_num(x), 0, W - 1)).astype(np.int64)
    row = np.floor(np.clip(np.nan_to_num(y), 0, H - 1)).astype(np.int64)
    exp = np.full((H, W, 8), NONE, dtype=np.uint32)
    ids = np.nonzero(ok)[0]
    for p in np.unique(row[ids] * W + col[ids]):
        mine = ids[(row[ids] * W + col[ids]) == p].astype(np.uint32)
        sc = orc.score_pairs(S, n, W, H, np.full(mine.size, p, dtype=np.uint32), mine)
        keep = mine[np.isfinite(sc)]
        sc = sc[np.isfinite(sc)]
        order = keep[np.lexsort((keep, sc))][:4]
        exp.reshape(-1, 8)[p, :order.size] = order
    return exp


def test_jfa_seed_definition(orc):
    W, H, n = 21, 13, 90
    S = synth.random_sites(n, W, H, 41)
    # a crowded pixel: six sites inside pixel (5, 4)
    S[synth.X, :6] = 5.0 + np.linspace(0.1, 0.9, 6)
    S[synth.Y, :6] = 4.0 + np.linspace(0.9, 0.1, 6)
    S[synth.X, 10] = -1.0           # inactive
    S[synth.X, 11] = np.nan         # no position
    S[synth.Y, 12] = np.inf
    S[synth.X, 13] = float(W)       # on the right border: the last column
    S[synth.Y, 14] = -3.0           # above the image: the first row
    S[synth.X, 15] = 1e6            # far right: the last column
    S[synth.X, 16] = 1e30           # so far that the float32 score overflows: dropped
    got = orc.jfa_seed(S, n, W, H)
    exp = _expected_seed(orc, S, n, W, H)
    assert np.array_equal(got, exp)
    assert (got[..., 4:] == NONE).all()
    lst = got[4, 5]
    assert (lst[:4] != NONE).all() and set(lst[:4].tolist()) <= set(range(6))
    assert got[..., :4].ravel().tolist().count(10) == 0 and 11 not in got and 12 not in got
    assert 13 in got[:, W - 1] and 15 in got[:, W - 1] and 14 in got[0] and 16 not in got


def test_jfa_pass_brute_force_union(orc):
    W, H, n = 17, 11, 70
    S = synth.random_sites(n, W, H, 42)
    S[synth.X, 3] = -1.0
    cin = synth.random_map(W, H, n + 3, seed=43)
    for step in (1, 2, 5, 16):
        out = orc.jfa_pass(S, n, cin, W, H, step).reshape(-1, 8)
        for p in range(W * H):
            r, c = divmod(p, W)
            cand = []
            for dr in (-step, 0, step):
                for dc in (-step, 0, step):
                    if 0 <= r + dr < H and 0 <= c + dc < W:
                        cand += list(cin[r + dr, c + dc, :4])
            ids = np.array(sorted({int(i) for i in cand if i < n and not S[synth.X, i] < 0}), dtype=np.uint32)
            sc = orc.score_pairs(S, n, W, H, np.full(ids.size, p, dtype=np.uint32), ids)
            ids, sc = ids[np.isfinite(sc)], sc[np.isfinite(sc)]
            order = ids[np.lexsort((ids, sc))][:4]
            exp = np.full(8, NONE, dtype=np.uint32)
            exp[:order.size] = order
            assert np.array_equal(out[p], exp), (step, p)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_jfa_few_sites_reach_every_pixel(orc, n):
    W, H = 37, 23
    S = synth.random_sites(n, W, H, 44 + n)
    m = orc.jfa_seed(S, n, W, H)
    for k in orc.jfa_steps(W, H):
        m = orc.jfa_pass(S, n, m, W, H, k)
    exact = orc.topk_exact(S, n, W, H)
    assert np.array_equal(m[..., :4], exact[..., :4])
    assert (m[..., 4:] == NONE).all()


def test_jfa_exact_top4_is_fixed_point(orc):
    W, H, n = 19, 15, 60
    S = synth.random_sites(n, W, H, 48)
    exact = orc.topk_exact(S, n, W, H)
    top4 = exact.copy()
    top4[..., 4:] = NONE
    for step in (1, 3, 8, 32):
        assert np.array_equal(orc.jfa_pass(S, n, top4, W, H, step), top4)


def test_jfa_euclidean_nearest_site(orc):
    from scipy.spatial import cKDTree

    W, H, n = 96, 64, 400
    S = synth.random_sites(n, W, H, 49)
    S[synth.A] = 0.0
    S[synth.R] = 0.0
    m = orc.jfa_seed(S, n, W, H)
    for k in orc.jfa_steps(W, H):
        m = orc.jfa_pass(S, n, m, W, H, k)
    rows, cols = np.divmod(np.arange(W * H), W)
    tree = cKDTree(np.stack([S[synth.X, :n], S[synth.Y, :n]], -1).astype(np.float64))
    dist, idx = tree.query(np.stack([cols + 0.5, rows + 0.5], -1), k=2)
    first = m.reshape(-1, 8)[:, 0]
    ties = dist[:, 1] - dist[:, 0] < 1e-5
    hit = (first == idx[:, 0]) | ties
    assert hit.mean() >= 0.99, hit.mean()


def test_jfa_steps():
    assert oracle.jfa_steps(768, 512) == [512, 256, 128, 64, 32, 16, 8, 4, 2, 1]
    assert len(oracle.jfa_steps(4096, 4096)) == 12 and len(oracle.jfa_steps(2040, 1356)) == 11
    assert oracle.jfa_steps(1, 1) == []
