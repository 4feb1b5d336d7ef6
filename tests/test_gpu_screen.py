"""The candidate screen (sad_site_screen, and the screen words sad_adam_step_rec
refreshes): a 4-byte word per site from which a selection pass proves that a
candidate scores after its list's K-th entry without fetching the candidate's
record.  It is an acceleration only, so:

* every word is checked against the definition: decoded in float64, the cell it
  names contains the site, 2^(ca/2) >= e^{|a|/2}, 2^(cr-8) >= 2^(ca/2) max(r, 0),
  and then for random points the distance bound implies d > the threshold used;
* propagation gives the same bits with and without it,
  on cold-start, mid-fit and edited maps, at small and large jumps, with
  injection, and with sites the word cannot bound (huge |a| or r, inactive,
  non-finite, outside the image);
* Adam's refreshed words equal sad_site_screen's on the updated sites.
"""
import numpy as np
import pytest
import torch

import soft_voronoi_render_amd as sad
import synth
from sadtest import map_to_host, to_dev

pytestmark = pytest.mark.gpu


def _sites(n, W, H, seed, cap=None, extreme=True):
    S = synth.random_sites(n, W, H, seed, cap)
    if extreme:
        rng = np.random.default_rng(seed)
        k = max(n // 20, 1)
        idx = rng.choice(n, 6 * k, replace=False)
        S[synth.A, idx[:k]] = rng.uniform(-12, 12, k)          # some beyond the word's range
        S[synth.R, idx[k:2 * k]] = rng.uniform(-5, 80, k)      # negative r, r past 64 px
        S[synth.X, idx[2 * k]] = -1.0                           # inactive
        S[synth.A, idx[2 * k + 1]] = np.nan
        S[synth.X, idx[3 * k:4 * k]] = np.floor(S[synth.X, idx[3 * k:4 * k]] * 4096 / W) * W / 4096  # on cell edges
        S[synth.X, idx[4 * k]] = W                               # on the image edge
        S[synth.Y, idx[4 * k + 1]] = H
        S[synth.DX, idx[5 * k]] = S[synth.DY, idx[5 * k]] = 0.0  # degenerate direction
    return S


def _screen(S, n, W, H):
    S_d = to_dev(S)
    scr = sad.new_screen(S.shape[1], S_d.device)
    sad.site_screen(S_d, n, W, H, scr)
    torch.cuda.synchronize()
    return scr, scr.cpu().numpy().view(np.uint32)[:n]


@pytest.mark.parametrize("W,H", [(64, 64), (77, 45), (2048, 2048), (4096, 4096), (65535, 3)])
def test_screen_words_bound_the_score(W, H):
    n = 3000
    S = _sites(n, W, H, 5)
    _, w = _screen(S, n, W, H)
    qx, qy = w & 0xFFF, (w >> 12) & 0xFFF
    ca, cr = (w >> 24) & 15, w >> 28
    x, y, r, a = (S[j, :n].astype(np.float64) for j in (synth.X, synth.Y, synth.R, synth.A))
    bounded = (ca != 15) & (cr != 15)
    ok = (x >= 0) & np.isfinite(x) & np.isfinite(y) & np.isfinite(a) & np.isfinite(r)
    assert not (bounded & ~ok).any(), "a site the word cannot bound got a bound"
    assert (~bounded[np.abs(np.nan_to_num(a, nan=99)) > 9.8]).all()
    cw, ch = W / 4096.0, H / 4096.0
    b = bounded
    eps = 1e-3 * max(cw, ch)
    assert (x[b] >= qx[b] * cw - eps).all() and (x[b] <= (qx[b] + 1) * cw + eps).all()
    assert (y[b] >= qy[b] * ch - eps).all() and (y[b] <= (qy[b] + 1) * ch + eps).all()
    Ahat = 2.0 ** (ca[b] / 2.0)
    assert (Ahat >= np.exp(np.abs(a[b]) / 2)).all()
    Rhat = np.where(cr[b] > 0, 2.0 ** (cr[b].astype(np.float64) - 8), 0.0)
    assert (Rhat >= Ahat * np.maximum(r[b], 0)).all()
    # the screen's test at random points implies d > kth for the exact score
    rng = np.random.default_rng(1)
    idx = np.nonzero(b)[0]
    s = 1.0 / max(W, H)
    dx_, dy_ = S[synth.DX, idx].astype(np.float64), S[synth.DY, idx].astype(np.float64)
    nrm = np.hypot(dx_, dy_)
    ux = np.where(nrm > 1e-15, dx_ / np.where(nrm > 0, nrm, 1), 1.0)
    uy = np.where(nrm > 1e-15, dy_ / np.where(nrm > 0, nrm, 1), 0.0)
    for _ in range(20):
        X = rng.uniform(0, W, idx.size)
        Y = rng.uniform(0, H, idx.size)
        kth = rng.uniform(-0.01, 0.05, idx.size)
        i = idx
        x0, y0 = qx[i] * cw, qy[i] * ch
        ddx = np.maximum(np.maximum(x0 - X, X - (x0 + cw)), 0)
        ddy = np.maximum(np.maximum(y0 - Y, Y - (y0 + ch)), 0)
        B = Ahat * np.maximum(kth, 0) / s + Rhat
        out = ddx ** 2 + ddy ** 2 > B ** 2
        ex, ey = X - x[i], Y - y[i]
        al, be = ux * ex + uy * ey, ux * ey - uy * ex
        d = s * np.sqrt(np.exp(a[i]) * al ** 2 + np.exp(-a[i]) * be ** 2) - s * r[i]
        assert (d[out] > kth[out]).all()


def _prop(rec, n, cin, W, H, jump, pidx, m, scr):
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device)
    sad.topk_propagate_rec(rec, n, a, b, W, H, jump, pidx, 13, m, scr=scr)
    torch.cuda.synchronize()
    return map_to_host(b)


@pytest.mark.parametrize("W,H,n", [(77, 45, 300), (130, 70, 2000), (256, 192, 20000), (1, 50, 40)])
def test_propagation_is_unchanged_by_the_screen(W, H, n):
    print(f"screen propagate W={W} H={H} n={n}", flush=True)
    S = _sites(n, W, H, 7)
    S_d = to_dev(S)
    rec = sad.new_records(n, S_d.device)
    sad.site_records(S_d, n, rec)
    scr, _ = _screen(S, n, W, H)
    maps = {"local": synth.local_map(S, n, W, H, seed=8, radius=5.0), "random": synth.random_map(W, H, n, seed=9),
            "empty": synth.empty_map(W, H)}
    for name, cin in maps.items():
        for jump, m in ((1, 4), (1, 16), (2, 8), (16, 4), (64, 8), (1000, 16)):
            with_scr = _prop(rec, n, cin, W, H, jump, 5, m, scr)
            without = _prop(rec, n, cin, W, H, jump, 5, m, None)
            assert np.array_equal(with_scr, without), f"{name} map, jump {jump}, {m} injected"
    # a schedule from the cold start, with and without
    a1 = a2 = synth.empty_map(W, H)
    for t, k in enumerate(sad.jump_schedule(W, H, 14)):
        a1 = _prop(rec, n, a1, W, H, k, t, 8, scr)
        a2 = _prop(rec, n, a2, W, H, k, t, 8, None)
        assert np.array_equal(a1, a2), f"schedule pass {t}"


def test_grid_passes_are_unchanged_by_the_screen():
    W, H, n = 203, 131, 5000
    S = _sites(n, W, H, 17)
    S_d = to_dev(S)
    rec = sad.new_records(n, S_d.device)
    sad.site_records(S_d, n, rec)
    scr, _ = _screen(S, n, W, H)
    for cell in (1, 3, 8):
        cin = map_to_host(sad.new_map(W, H, cell=cell))
        for t, k in enumerate(sad.jump_schedule(W, H, 10, cell=cell)):
            res = []
            for sc in (scr, None):
                a = to_dev(cin)
                b = sad.new_map(W, H, a.device, cell)
                sad.topk_propagate_rec(rec, n, a, b, W, H, k, t, 3, 4, cell=cell, scr=sc)
                torch.cuda.synchronize()
                res.append(map_to_host(b))
            assert np.array_equal(res[0], res[1]), f"cell {cell}, pass {t}"
            cin = res[1]


def test_edited_map_refresh_is_unchanged_by_the_screen():
    """The edit-stress pattern at 1024x1024 with 64k sites: converge, move 10 % of
    the sites by up to 256 px, refresh with 8 injected per pixel."""
    W, H, n = 1024, 1024, 65536
    S = synth.random_sites(n, W, H, 21)
    S_d = to_dev(S)
    rec = sad.new_records(n, S_d.device)
    sad.site_records(S_d, n, rec)
    scr = sad.new_screen(n, S_d.device)
    sad.site_screen(S_d, n, W, H, scr)
    a, b = sad.new_map(W, H), sad.new_map(W, H)
    sched = sad.jump_schedule(W, H, 10)
    for t, k in enumerate(sched + [1] * 6):
        sad.topk_propagate_rec(rec, n, a, b, W, H, k, t, 4, 8, scr=scr)
        a, b = b, a
    S2 = synth.displace_sites(S, n, W, H, seed=77)
    S_d.copy_(torch.from_numpy(S2))
    sad.site_records(S_d, n, rec)
    sad.site_screen(S_d, n, W, H, scr)
    start = a.clone()
    res = []
    for sc in (scr, None):
        x, y = start.clone(), sad.new_map(W, H)
        for t, k in enumerate(sched):
            sad.topk_propagate_rec(rec, n, x, y, W, H, k, 100 + t, 4, 8, scr=sc)
            x, y = y, x
        torch.cuda.synchronize()
        res.append(map_to_host(x))
    assert np.array_equal(res[0], res[1])


def test_adam_refreshes_the_screen():
    W, H, n, cap = 300, 200, 4000, 4100
    S = _sites(n, W, H, 31, cap)
    S_d = to_dev(S)
    m = torch.zeros((10, cap), dtype=torch.float32, device=S_d.device)
    v = torch.zeros_like(m)
    g = torch.from_numpy(np.random.default_rng(2).normal(0, 500, (cap, 16)).astype(np.float32)).to(S_d.device)
    scr = sad.new_screen(cap, S_d.device)
    sad.adam_step_rec(S_d, m, v, g, n, 1, W * H, W, H, scr=scr)
    fresh = sad.new_screen(cap, S_d.device)
    sad.site_screen(S_d, n, W, H, fresh)
    torch.cuda.synchronize()
    assert torch.equal(scr[:n], fresh[:n])
    assert (scr[n:] == 0).all()
