"""GPU parity of the iteration on the site buffer -- sad_topk_propagate,
sad_render_fwd, sad_render_bwd and sad_adam_step, which read the ten site planes
directly and write eleven gradient planes and a scalar loss -- through the C ABI,
against the CPU oracle on the same seeded inputs (ragged multi-tile sizes and the
edge cases of the method), and against the cached calls (*_rec) on the same
sites: the selection, the images and the Adam update must be the same bits, the
gradients equal within the float-atomic order."""
import numpy as np
import pytest
import torch

import soft_voronoi_render_amd as sad
import synth
from oracle.densify import densify_prune as orc_densify
from sadtest import FWD_TOL, GRAD_TOL, NONE, compare_lists, map_to_host, rel_l2, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(64, 64, 256), (77, 45, 300), (1, 1, 3), (33, 1, 20), (1, 50, 40), (130, 70, 2000)]


def _case(W, H, n, seed=1, stride=None):
    S = synth.random_sites(n, W, H, seed, stride)
    cin = synth.local_map(S, n, W, H, seed=seed + 10, radius=6.0)
    return S, cin


def _rec(S_d, n):
    g = sad.new_records(S_d.shape[1], S_d.device)
    sad.site_records(S_d, n, g)
    return g


@pytest.mark.parametrize("W,H,n", SHAPES)
@pytest.mark.parametrize("jump,m", [(1, 4), (5, 0), (64, 8), (1000, 16)])
def test_propagate_from_the_planes(orc, W, H, n, jump, m):
    print(f"site-buffer propagate W={W} H={H} n={n} jump={jump} m={m}", flush=True)
    S, cin = _case(W, H, n, stride=n + 7)  # stride > n_slots
    S_d = to_dev(S)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device)
    sad.topk_propagate(S_d, n, a, b, W, H, jump, 4321, 99, m)
    c = sad.new_map(W, H, a.device)
    sad.topk_propagate_rec(_rec(S_d, n), n, a, c, W, H, jump, 4321, 99, m)
    torch.cuda.synchronize()
    got = map_to_host(b)
    assert np.array_equal(got, map_to_host(c)), "planes and records select differently"
    ref = orc.propagate(S, n, cin, W, H, jump, 4321, 99, m)
    pix = np.arange(W * H)
    u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 4321, 99, m, pix)
    assert compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt) <= max(2, W * H // 2000)


def test_propagate_from_the_planes_edge_inputs(orc):
    """Sentinels, IDs >= n_slots, inactive, NaN and duplicate sites, N < K, n_slots
    = 0, an all-sentinel map with injection only."""
    W, H, n = 40, 24, 60
    S = synth.random_sites(n, W, H, 3)
    S[synth.X, 5] = -1.0
    S[synth.X, 7] = np.nan
    S[synth.A, 9] = np.nan
    S_d = to_dev(S)
    pix = np.arange(W * H)
    for cin, nn, jump, m in [(synth.random_map(W, H, n + 5, seed=4, p_invalid=0.3, p_dup=0.3), n, 2, 6),
                             (synth.random_map(W, H, n, seed=5), 4, 1, 3),
                             (synth.random_map(W, H, n, seed=6), 0, 1, 4),
                             (synth.empty_map(W, H), n, 32, 4)]:
        a = to_dev(cin)
        b = sad.new_map(W, H, a.device)
        sad.topk_propagate(S_d, nn, a, b, W, H, jump, 17, 5, m)
        torch.cuda.synchronize()
        got = map_to_host(b)
        ref = orc.propagate(S, nn, cin, W, H, jump, 17, 5, m)
        u, cnt = orc.union_pixels(S, nn, cin, W, H, jump, 17, 5, m, pix)
        assert compare_lists(orc, S, nn, W, H, pix, got, ref, u, cnt) <= 1


@pytest.mark.parametrize("W,H,n", SHAPES)
def test_render_fwd_from_the_planes(orc, W, H, n):
    S, cin = _case(W, H, n, seed=2, stride=n + 3)
    cand = orc.propagate(S, n, cin, W, H, 1, 0, 1, 4)
    S_d, c = to_dev(S), to_dev(cand)
    out = torch.empty((H, W, 3), dtype=torch.float32, device=S_d.device)
    sad.render_fwd(S_d, n, c, W, H, out)
    ref_rec = torch.empty_like(out)
    sad.render_fwd_rec(_rec(S_d, n), n, c, W, H, ref_rec)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, ref_rec.cpu().numpy())
    assert np.abs(got - orc.render_fwd(S, n, cand, W, H)).max() <= FWD_TOL


def _bwd_planes(S, n, cand, tgt, W, H, grad0=None):
    S_d = to_dev(S)
    g = sad.new_grad_planes(S.shape[1], S_d.device)
    if grad0 is not None:
        g.copy_(torch.from_numpy(grad0))
    loss = torch.zeros(1, dtype=torch.float32, device=S_d.device)
    sad.render_bwd(S_d, n, to_dev(cand), to_dev(tgt), W, H, g, loss)
    torch.cuda.synchronize()
    return g.cpu().numpy().astype(np.float64), float(loss.item())


def _check(got, ref, n):
    for j in range(11):
        r = rel_l2(got[j, :n], ref[j, :n])
        assert r <= GRAD_TOL, f"plane {j}: rel L2 {r:.3e}"


@pytest.mark.parametrize("W,H,n", SHAPES)
def test_render_bwd_into_planes(orc, W, H, n):
    print(f"site-buffer bwd W={W} H={H} n={n}", flush=True)
    S, cin = _case(W, H, n, seed=3, stride=n + 5)
    cand = orc.propagate(S, n, cin, W, H, 1, 0, 1, 4)
    tgt = orc.hard_render(synth.random_sites(n, W, H, 33), n, W, H) + synth.pixel_noise(W, H, 5)
    got, loss = _bwd_planes(S, n, cand, tgt, W, H)
    ref, rloss = orc.render_bwd(S, n, cand, tgt, W, H)
    _check(got, ref, n)
    assert (got[:, n:] == 0).all(), "slots beyond n_slots were written"
    assert loss == pytest.approx(rloss, rel=1e-4)


def test_render_bwd_into_planes_overflow_and_edges(orc):
    """A tile naming far more sites than its table holds (global-atomic path),
    then inactive, non-finite, degenerate and sole-contributor entries with
    accumulation onto existing planes."""
    W, H, n = 64, 48, 20000
    S = synth.random_sites(n, W, H, 11)
    cand = synth.random_map(W, H, n, seed=12, p_invalid=0.0, p_dup=0.0)
    tgt = synth.pixel_noise(W, H, 6, 0.3) + 0.5
    got, loss = _bwd_planes(S, n, cand, tgt, W, H)
    ref, rloss = orc.render_bwd(S, n, cand, tgt, W, H)
    _check(got, ref, n)
    assert loss == pytest.approx(rloss, rel=1e-4)
    W, H, n = 35, 19, 80
    S = synth.random_sites(n, W, H, 13)
    S[synth.X, 2] = -1.0
    S[synth.CG, 3] = np.inf
    S[synth.DX, 4] = S[synth.DY, 4] = 0.0
    S[synth.X, 5], S[synth.Y, 5] = 10.5, 7.5
    cand = synth.random_map(W, H, n + 2, seed=14, p_invalid=0.25, p_dup=0.1)
    cand[3, :, :] = NONE
    cand[7, 10, :] = [5, NONE, NONE, NONE, NONE, NONE, NONE, NONE]
    tgt = synth.pixel_noise(W, H, 7, 0.3) + 0.5
    g0 = np.random.default_rng(0).normal(0, 1, (11, n)).astype(np.float32)
    got, loss = _bwd_planes(S, n, cand, tgt, W, H, grad0=g0)
    ref, rloss = orc.render_bwd(S, n, cand, tgt, W, H, grad=g0.astype(np.float64))
    _check(got, ref, n)
    assert np.isfinite(got).all()
    assert loss == pytest.approx(rloss, rel=1e-4)


@pytest.mark.parametrize("step", [1, 7, 1000])
def test_adam_on_planes(orc, step):
    W, H, n, cap = 100, 80, 700, 777
    S = synth.random_sites(n, W, H, 15, cap)
    S[synth.X, 10] = -1.0
    S[synth.X, 11] = 0.01
    rng = np.random.default_rng(step)
    m = rng.normal(0, 1e-3, (10, cap)).astype(np.float32)
    v = (rng.random((10, cap)) * 1e-5).astype(np.float32)
    G = rng.normal(0, 50, (11, cap)).astype(np.float32)
    G[0, 11] = 1e6
    G[3, 12] = np.nan
    cfg = sad.AdamConfig()
    S_d, m_d, v_d, G_d = (to_dev(a) for a in (S, m, v, G))
    sad.adam_step(S_d, m_d, v_d, G_d, n, step, W * H, W, H, cfg)
    # the cached call on the same inputs (gradient records)
    S2, m2, v2 = (to_dev(a) for a in (S, m, v))
    rec = np.zeros((cap, 16), dtype=np.float32)
    rec[:, :11] = G.T
    R_d = to_dev(rec)
    sad.adam_step_rec(S2, m2, v2, R_d, n, step, W * H, W, H, cfg)
    torch.cuda.synchronize()
    for a, b in ((S_d, S2), (m_d, m2), (v_d, v2)):
        assert torch.equal(a, b)
    Gh = G_d.cpu().numpy()
    assert (Gh[:10, :n] == 0).all() and np.array_equal(Gh[:10, n:], G[:10, n:])
    assert np.array_equal(Gh[10], G[10]), "the removal plane is left alone"
    p64, m64, v64, g64 = (a.astype(np.float64) for a in (S, m, v, G))
    f32 = lambda x: float(np.float32(x))
    orc.adam_step(p64, m64, v64, g64, n, step, W * H, np.array(cfg.lr, dtype=np.float32).astype(np.float64),
                  f32(cfg.beta1), f32(cfg.beta2), f32(cfg.eps), W, H)
    for a, b in zip((S_d, m_d, v_d), (p64, m64, v64)):
        assert np.allclose(a.cpu().numpy().astype(np.float64), b, rtol=1e-5, atol=1e-7)
    assert S_d[0, 11].item() == 0.0


def test_site_buffer_iteration_chain(orc):
    """Nine warm-up iterations through the site-buffer calls (propagate, render
    forward, render backward, Adam; budget control after the second) on a coherent
    fit state.  The state is the oracle's: every GPU call gets the oracle's current
    state as input and its output is compared with the oracle's step, which then
    advances the state."""
    W, H, n, cap = 80, 56, 400, 440
    S = synth.random_sites(n, W, H, 41, cap)
    tgt = (orc.hard_render(synth.random_sites(n, W, H, 42), n, W, H) + synth.pixel_noise(W, H, 43)).astype(
        np.float32)
    t_d = to_dev(tgt)
    p64 = S.astype(np.float64)
    m64, v64 = np.zeros((10, cap)), np.zeros((10, cap))
    G = np.zeros((11, cap))
    cand = synth.empty_map(W, H)
    pix = np.arange(W * H)
    cfg = sad.AdamConfig()
    f32 = lambda x: float(np.float32(x))
    lr = np.array(cfg.lr, dtype=np.float32).astype(np.float64)
    for it, jump in enumerate(sad.jump_schedule(W, H, 9)):
        S32 = p64.astype(np.float32)
        S_d = to_dev(S32)
        a, b = to_dev(cand), sad.new_map(W, H)
        sad.topk_propagate(S_d, n, a, b, W, H, jump, it, 7, 4)
        torch.cuda.synchronize()
        ref = orc.propagate(S32, n, cand, W, H, jump, it, 7, 4)
        u, cnt = orc.union_pixels(S32, n, cand, W, H, jump, it, 7, 4, pix)
        assert compare_lists(orc, S32, n, W, H, pix, map_to_host(b), ref, u, cnt) <= 2
        cand = ref
        c_d = to_dev(cand)
        rgb = torch.empty((H, W, 3), dtype=torch.float32, device=S_d.device)
        sad.render_fwd(S_d, n, c_d, W, H, rgb)
        g_d = to_dev(G.astype(np.float32))
        loss = torch.zeros(1, dtype=torch.float32, device=S_d.device)
        sad.render_bwd(S_d, n, c_d, t_d, W, H, g_d, loss)
        torch.cuda.synchronize()
        assert np.abs(rgb.cpu().numpy() - orc.render_fwd(S32, n, cand, W, H)).max() <= FWD_TOL
        G, lref = orc.render_bwd(S32, n, cand, tgt, W, H, grad=G.astype(np.float32).astype(np.float64))
        _check(g_d.cpu().numpy().astype(np.float64), G, n)
        assert loss.item() == pytest.approx(lref, rel=1e-4)
        # Adam from the oracle's state and gradients
        P_d, M_d, V_d, G_d = (to_dev(x.astype(np.float32)) for x in (p64, m64, v64, G))
        sad.adam_step(P_d, M_d, V_d, G_d, n, it + 1, W * H, W, H, cfg)
        torch.cuda.synchronize()
        p64, m64, v64, G = (x.astype(np.float32).astype(np.float64) for x in (p64, m64, v64, G))
        orc.adam_step(p64, m64, v64, G, n, it + 1, W * H, lr, f32(cfg.beta1), f32(cfg.beta2), f32(cfg.eps), W, H)
        for x_d, x in ((P_d, p64), (M_d, m64), (V_d, v64), (G_d, G)):
            assert np.allclose(x_d.cpu().numpy().astype(np.float64), x, rtol=1e-5, atol=1e-7)
        if it == 1:
            # budget control: the library's host routine on the oracle's state vs the
            # oracle's statistics and rules
            bc = sad.BudgetConfig(split_frac=0.05, prune_frac=0.05)
            S32 = p64.astype(np.float32)
            mine = [S32.copy(), m64.astype(np.float32), v64.astype(np.float32), G[10].astype(np.float32),
                    cand.copy()]
            n2, rc = sad.densify_prune(mine[0], mine[1], mine[2], mine[3], n, cap, mine[4], W, H, tgt, bc)
            refs = [S32.copy(), m64.astype(np.float32), v64.astype(np.float32), G[10].astype(np.float32),
                    cand.copy()]
            st = orc.densify_stats(S32, n, cand, tgt, W, H).astype(np.float32)
            want = orc_densify(refs[0], refs[1], refs[2], n, cap, st, refs[3], refs[4], W, H, tgt,
                               f32(bc.split_frac), f32(bc.prune_frac), f32(bc.alpha), f32(bc.min_mass),
                               f32(bc.shrink))
            assert rc == 0 and n2 == want[0] and want[1] > 0
            assert np.allclose(mine[0], refs[0], atol=2e-5, equal_nan=True)
            assert np.array_equal(mine[4], refs[4])
            assert np.all(mine[3][:n2] == 0)
            n = n2
            p64, m64, v64 = (x.astype(np.float64) for x in refs[:3])
            G[10] = 0.0
            cand = refs[4]
            for lst in cand.reshape(-1, 8):
                v_ = lst[lst != NONE]
                assert len(set(v_.tolist())) == v_.size
