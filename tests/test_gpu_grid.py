"""GPU parity of the downscaled candidate grid (paperlayer.ai summary, Appendix B.3
"Candidate field") through the C ABI: every entry point that reads or writes the
map, with cells of c x c pixels, against the oracle on the same seeded inputs.

Selection (exact top-8, propagation with injection, the jump-flood seed and
flood passes) runs over the ceil(W/c) x ceil(H/c) map entries and scores at the
centred cell UV; the render, its backward and the budget statistics evaluate
every pixel at its own centre with the list of its cell.  Sizes span several
tiles with ragged tails, cells that divide neither W nor H, a one-row image and
a cell larger than the image.  The last test runs the kodak768 fit with c = 4
and reports the time per iteration and the PSNR next to the per-pixel map.
"""
import numpy as np
import pytest
import torch

import soft_voronoi_render_amd as sad
import synth
from sadtest import FWD_TOL, GRAD_TOL, NONE, compare_lists, map_to_host, rel_l2, to_dev

pytestmark = pytest.mark.gpu

# (W, H, n, cell)
CASES = [(64, 64, 256, 2), (77, 45, 300, 4), (130, 70, 2000, 3), (33, 1, 20, 4), (5, 3, 6, 8),
         (200, 120, 1500, 16)]


def _rec(S, n):
    S_d = to_dev(S)
    g = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, g)
    return g


def _entries(W, H, c):
    Hm, Wm, _ = sad.map_shape(W, H, c)
    return np.arange(Wm * Hm, dtype=np.uint32)


def _sites(n, W, H, seed):
    S = synth.random_sites(n, W, H, seed, n + 3)
    if n >= 20:
        S[synth.X, 3] = -1.0          # inactive
        S[synth.X, 5] = float(W) + 2  # beyond the right border
        S[synth.Y, 6] = np.nan        # no position
    return S


@pytest.mark.parametrize("W,H,n,c", CASES)
def test_grid_topk_exact(orc, W, H, n, c):
    print(f"grid exact W={W} H={H} n={n} c={c}", flush=True)
    S = _sites(n, W, H, 71)
    g = _rec(S, n)
    out = sad.new_map(W, H, g.device, cell=c)
    sad.topk_exact(g, n, out, W, H, cell=c)
    torch.cuda.synchronize()
    got = map_to_host(out)
    ref = orc.topk_exact(S, n, W, H, cell=c)
    assert got.shape == ref.shape
    pix = _entries(W, H, c)
    assert compare_lists(orc, S, n, W, H, pix, got, ref, cell=c) <= max(1, pix.size // 2000)


@pytest.mark.parametrize("W,H,n,c", CASES)
@pytest.mark.parametrize("jump,m", [(1, 4), (2, 0), (8, 8)])
def test_grid_propagate(orc, W, H, n, c, jump, m):
    print(f"grid propagate W={W} H={H} n={n} c={c} jump={jump} m={m}", flush=True)
    S = _sites(n, W, H, 72)
    Hm, Wm, _ = sad.map_shape(W, H, c)
    cin = synth.random_map(Wm, Hm, n + 3, seed=73)
    g = _rec(S, n)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device, cell=c)
    sad.topk_propagate_rec(g, n, a, b, W, H, jump, 999, 31, m, cell=c)
    torch.cuda.synchronize()
    got = map_to_host(b)
    ref = orc.propagate(S, n, cin, W, H, jump, 999, 31, m, cell=c)
    pix = _entries(W, H, c)
    u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 999, 31, m, pix, cell=c)
    assert compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt, cell=c) <= max(2, pix.size // 2000)


@pytest.mark.parametrize("jump", [1, 16])
def test_grid_propagate_large_map(orc, jump):
    """A map of more than a thousand 16x16 tiles (515 x 515 entries of 2 x 2
    pixels): the launch shape large grid maps take."""
    W, H, n, c = 1030, 1030, 20000, 2
    print(f"grid propagate large map jump={jump}", flush=True)
    S = _sites(n, W, H, 79)
    Hm, Wm, _ = sad.map_shape(W, H, c)
    cin = orc.topk_exact(S, n, W, H, cell=4)  # coherent lists from a coarser grid
    cin = np.ascontiguousarray(cin[np.arange(Hm) // 2][:, np.arange(Wm) // 2])
    g = _rec(S, n)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device, cell=c)
    sad.topk_propagate_rec(g, n, a, b, W, H, jump, 321, 9, 4, cell=c)
    torch.cuda.synchronize()
    got = map_to_host(b)
    ref = orc.propagate(S, n, cin, W, H, jump, 321, 9, 4, cell=c)
    pix = _entries(W, H, c)
    mism = np.nonzero((got.reshape(-1, 8) != ref.reshape(-1, 8)).any(1))[0].astype(np.uint32)
    u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 321, 9, 4, mism, cell=c)
    bad = compare_lists(orc, S, n, W, H, mism, got.reshape(-1, 8)[mism], ref.reshape(-1, 8)[mism], u, cnt, cell=c)
    assert bad <= pix.size // 2000


@pytest.mark.parametrize("W,H,n,c", CASES)
def test_grid_jfa(orc, W, H, n, c):
    print(f"grid jfa W={W} H={H} n={n} c={c}", flush=True)
    S = _sites(n, W, H, 74)
    g = _rec(S, n)
    a = sad.new_map(W, H, g.device, cell=c)
    a.fill_(7)
    sad.jfa_seed(g, n, a, W, H, cell=c)
    torch.cuda.synchronize()
    seed_map = map_to_host(a)
    ref = orc.jfa_seed(S, n, W, H, cell=c)
    pix = _entries(W, H, c)
    assert (seed_map[..., 4:] == NONE).all()
    bad = compare_lists(orc, S, n, W, H, pix, seed_map, ref, cell=c)
    cur = ref
    for k in sad.jfa_steps(W, H, cell=c)[-3:]:
        x = to_dev(cur)
        y = sad.new_map(W, H, x.device, cell=c)
        sad.jfa_pass(g, n, x, y, W, H, k, cell=c)
        torch.cuda.synchronize()
        got = map_to_host(y)
        ref = orc.jfa_pass(S, n, cur, W, H, k, cell=c)
        u, cnt = orc.jfa_union_pixels(S, n, cur, W, H, k, pix, cell=c)
        bad += compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt, cell=c)
        cur = ref
    assert bad <= max(2, pix.size // 1000)


def _render_case(W, H, n, c, seed, random_lists):
    S = synth.random_sites(n, W, H, seed, n + 3)
    S[synth.X, n // 2] = -1.0
    Hm, Wm, _ = sad.map_shape(W, H, c)
    if random_lists:
        cand = synth.random_map(Wm, Hm, n + 3, seed=seed + 1, p_invalid=0.2, p_dup=0.2)
    else:
        cand = None  # filled by the caller with the oracle's exact lists
    tgt = (synth.pixel_noise(W, H, seed + 2, 0.2) + 0.5).astype(np.float32)
    return S, cand, tgt


@pytest.mark.parametrize("W,H,n,c", CASES)
@pytest.mark.parametrize("random_lists", [False, True])
def test_grid_render_fwd_bwd(orc, W, H, n, c, random_lists):
    print(f"grid render W={W} H={H} n={n} c={c} random={random_lists}", flush=True)
    S, cand, tgt = _render_case(W, H, n, c, 75, random_lists)
    if cand is None:
        cand = orc.topk_exact(S, n, W, H, cell=c)
    R = _rec(S, n)
    c_d = to_dev(cand)
    t_d = to_dev(tgt)
    out = torch.empty((H, W, 3), dtype=torch.float32, device=R.device)
    sad.render_fwd_rec(R, n, c_d, W, H, out, cell=c)
    g = sad.new_grad(S.shape[1], R.device)
    loss = sad.new_loss(R.device)
    rgb = torch.full((H, W, 3), -7.0, dtype=torch.float32, device=R.device)
    sad.render_bwd_rec(R, n, c_d, t_d, W, H, g, loss, rgb, cell=c)
    torch.cuda.synchronize()
    fwd = out.cpu().numpy()
    ref = orc.render_fwd(S, n, cand, W, H, cell=c)
    assert np.abs(fwd - ref).max() <= FWD_TOL
    assert np.array_equal(rgb.cpu().numpy(), fwd)
    gh = g.cpu().numpy().astype(np.float64)
    assert (gh[:, 11:] == 0).all()
    rg, rloss = orc.render_bwd(S, n, cand, tgt, W, H, cell=c)
    for j in range(11):
        r = rel_l2(gh[:, j], rg[j])
        assert r <= GRAD_TOL, f"plane {j}: rel L2 {r:.3e}"
    assert loss.sum().item() == pytest.approx(rloss, rel=1e-4)


@pytest.mark.parametrize("W,H,n,c", CASES)
def test_grid_densify_stats(orc, W, H, n, c):
    S, cand, tgt = _render_case(W, H, n, c, 76, True)
    R = _rec(S, n)
    st = torch.zeros((S.shape[1], sad.STAT_LD), dtype=torch.float32, device=R.device)
    sad.densify_stats(R, n, to_dev(cand), to_dev(tgt), W, H, st, cell=c)
    torch.cuda.synchronize()
    got = st.cpu().numpy().astype(np.float64)
    ref = orc.densify_stats(S, n, cand, tgt, W, H, cell=c)
    for a in range(7):
        assert rel_l2(got[:n, a], ref[:n, a]) <= GRAD_TOL, a
    assert (got[:, 7] == 0).all()


def test_grid_full_size_kodak768(orc):
    """kodak768 with cells of 4 pixels (192 x 128 lists), in the launch configuration
    of a fit step: the propagation pass at jump 1 on sampled entries and the fused
    forward+backward on the whole image, against the oracle."""
    wl = synth.WORKLOADS["kodak768"]
    W, H, n, c = wl.W, wl.H, wl.n_sites, 4
    S = synth.random_sites(n, W, H, 77, wl.capacity)
    Hm, Wm, _ = sad.map_shape(W, H, c)
    # coherent lists: the oracle's exact lists of a cell grid twice as coarse,
    # expanded, then one oracle propagation pass with injection
    coarse = orc.topk_exact(S, n, W, H, cell=2 * c)
    cin = np.ascontiguousarray(coarse[np.arange(Hm) // 2][:, np.arange(Wm) // 2])
    R = _rec(S, n)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device, cell=c)
    sad.topk_propagate_rec(R, n, a, b, W, H, 1, 5, synth.SEED_INJECT, wl.n_inject, cell=c)
    torch.cuda.synchronize()
    got = map_to_host(b).reshape(-1, 8)
    pix = np.unique(np.random.default_rng(5).choice(Wm * Hm, 6000, replace=False)).astype(np.uint32)
    ref = orc.propagate_pixels(S, n, cin, W, H, 1, 5, synth.SEED_INJECT, wl.n_inject, pix, cell=c)
    u, cnt = orc.union_pixels(S, n, cin, W, H, 1, 5, synth.SEED_INJECT, wl.n_inject, pix, cell=c)
    assert compare_lists(orc, S, n, W, H, pix, got[pix], ref, u, cnt, cell=c) <= 3
    cand = orc.propagate(S, n, cin, W, H, 1, 5, synth.SEED_INJECT, wl.n_inject, cell=c)
    tgt = (synth.pixel_noise(W, H, 78, 0.2) + 0.5).astype(np.float32)
    g = sad.new_grad(S.shape[1], R.device)
    loss = sad.new_loss(R.device)
    rgb = torch.empty((H, W, 3), dtype=torch.float32, device=R.device)
    sad.render_bwd_rec(R, n, to_dev(cand), to_dev(tgt), W, H, g, loss, rgb, cell=c)
    torch.cuda.synchronize()
    pp = np.unique(np.random.default_rng(6).choice(W * H, 20000, replace=False)).astype(np.uint32)
    fwd_ref = orc.render_fwd_pixels(S, n, cand, W, H, pp, cell=c)
    assert np.abs(rgb.cpu().numpy().reshape(-1, 3)[pp] - fwd_ref).max() <= FWD_TOL
    rg, rloss = orc.render_bwd(S, n, cand, tgt, W, H, cell=c)
    gh = g.cpu().numpy().astype(np.float64)
    for j in range(11):
        assert rel_l2(gh[:, j], rg[j]) <= GRAD_TOL, j
    assert loss.sum().item() == pytest.approx(rloss, rel=1e-4)


def test_grid_kodak768_fit():
    """The 200-iteration kodak768 fit with the per-pixel map and with cells of 2 and
    4 pixels: time per iteration and final PSNR, reported.  The grid fits must
    converge (the pages give no PSNR for a given cell size) and a coarser map must
    not be slower."""
    import bench

    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    S, tgt = bench.make_inputs(wl, torch.device("cuda:0"))
    res = {}
    for c in (1, 2, 4):
        f = sad.Fitter(to_dev(S), n, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT, cell=c)
        f.loss.zero_()
        f.step()
        torch.cuda.synchronize()
        psnr0 = 10 * np.log10(3 * W * H / f.loss.sum().item())
        f = sad.Fitter(to_dev(S), n, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT, cell=c)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(wl.iters):
            f.step()
        e1.record()
        f.loss.zero_()
        f.step()
        torch.cuda.synchronize()
        psnr = 10 * np.log10(3 * W * H / f.loss.sum().item())
        res[c] = (psnr, e0.elapsed_time(e1) / wl.iters)
        print(f"kodak768 cell {c}: PSNR {psnr0:.3f} -> {psnr:.3f} dB, {res[c][1] * 1e3:.1f} us per iteration",
              flush=True)
        assert psnr > psnr0 + 1.0
    assert res[4][1] <= res[1][1] * 1.05
