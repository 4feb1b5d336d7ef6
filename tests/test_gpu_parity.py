"""GPU parity: every libsad entry point, called through the C ABI, against the
CPU oracle on the same seeded inputs (small, multi-tile sizes with ragged tails
and edge cases; the full workload sizes are in test_gpu_fullsize.py)."""
import numpy as np
import pytest
import torch

import soft_voronoi_render_amd as sad
import synth
from sadtest import FWD_TOL, GRAD_TOL, NONE, compare_lists, map_to_host, rel_l2, to_dev

pytestmark = pytest.mark.gpu

# (W, H, n): several 16x16 tiles with ragged tails, a 1-pixel row, a thin column
SHAPES = [(64, 64, 256), (77, 45, 300), (1, 1, 3), (33, 1, 20), (1, 50, 40), (130, 70, 2000)]


def _case(W, H, n, seed=1):
    S = synth.random_sites(n, W, H, seed)
    cin = synth.local_map(S, n, W, H, seed=seed + 10, radius=6.0)
    return S, cin


def _rec(S, n):
    S_d = to_dev(S)
    g = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, g)
    return g


def _gpu_propagate(S, n, cin, W, H, jump, pidx, seed, m):
    g = _rec(S, n)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device)
    sad.topk_propagate_rec(g, n, a, b, W, H, jump, pidx, seed, m)
    torch.cuda.synchronize()
    return map_to_host(b)


@pytest.mark.parametrize("W,H,n", SHAPES)
@pytest.mark.parametrize("jump,m", [(1, 4), (2, 8), (3, 0), (7, 4), (16, 8), (1000, 16)])
def test_propagate_matches_oracle(orc, W, H, n, jump, m):
    print(f"propagate W={W} H={H} n={n} jump={jump} m={m}", flush=True)
    S, cin = _case(W, H, n)
    got = _gpu_propagate(S, n, cin, W, H, jump, 12345, 77, m)
    ref = orc.propagate(S, n, cin, W, H, jump, 12345, 77, m)
    pix = np.arange(W * H)
    u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 12345, 77, m, pix)
    bad = compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt)
    assert bad <= max(2, W * H // 2000)


def test_propagate_edge_inputs(orc):
    """Sentinels, IDs >= n_slots, inactive sites, duplicate IDs, NaN sites, N < K,
    n_slots = 0, and the 16-bit wrap of the pass index."""
    W, H, n = 40, 24, 60
    S = synth.random_sites(n, W, H, 3)
    S[synth.X, 5] = -1.0
    S[synth.X, 7] = np.nan
    S[synth.A, 9] = np.nan
    cin = synth.random_map(W, H, n + 5, seed=4, p_invalid=0.3, p_dup=0.3)
    for (nn, pidx) in [(n, 3), (n, 3 + 65536), (4, 9), (0, 1)]:
        got = _gpu_propagate(S, nn, cin, W, H, 2, pidx, 5, 6)
        ref = orc.propagate(S, nn, cin, W, H, 2, pidx, 5, 6)
        pix = np.arange(W * H)
        u, cnt = orc.union_pixels(S, nn, cin, W, H, 2, pidx, 5, 6, pix)
        assert compare_lists(orc, S, nn, W, H, pix, got, ref, u, cnt) <= 1
    assert np.array_equal(_gpu_propagate(S, n, cin, W, H, 2, 3, 5, 6), _gpu_propagate(S, n, cin, W, H, 2, 3 + 65536, 5, 6))


@pytest.mark.parametrize("seed,jump", [(21, 1), (22, 1), (23, 2), (24, 3), (25, 4), (26, 5), (27, 8)])
def test_propagate_table_overflow(orc, seed, jump):
    """Lists of uniformly random sites at the jumps whose pass keeps a 256-slot
    tile table: every tile names far more sites than the table holds, so own,
    neighbour and strip entries take the spill path (their IDs read again from
    the input map); sentinels and duplicates mixed in."""
    W, H, n = 67, 45, 20000
    print(f"propagate overflow jump={jump} seed={seed}", flush=True)
    S = synth.random_sites(n, W, H, seed)
    cin = synth.random_map(W, H, n, seed=seed + 1, p_invalid=0.1, p_dup=0.1)
    got = _gpu_propagate(S, n, cin, W, H, jump, 31, 77, 4)
    ref = orc.propagate(S, n, cin, W, H, jump, 31, 77, 4)
    pix = np.arange(W * H)
    u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 31, 77, 4, pix)
    assert compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt) <= 2


@pytest.mark.parametrize("jump", [5, 8, 16, 32, 48])
def test_propagate_five_region_table_overflow(orc, jump):
    """Tiles alternate between lists drawn from a pool of 40 sites (coherent own
    lists: the five-region table is used) and uniformly random lists. At these
    jumps a pool tile's neighbour regions are random tiles naming thousands of
    sites, so the key table runs out of probes (IDs read again as spills) and,
    with the sparse hash, more keys are occupied than there are records (the
    IDs beyond the last record also become spills)."""
    W, H, n = 96, 96, 20000
    print(f"propagate five-region overflow jump={jump}", flush=True)
    S = synth.random_sites(n, W, H, 41)
    cin = synth.random_map(W, H, n, seed=42, p_invalid=0.05, p_dup=0.05)
    rng = np.random.default_rng(43)
    for ty in range(H // 16):
        for tx in range(W // 16):
            if (tx + ty) % 2 == 0:
                pool = rng.choice(n, 40, replace=False)
                for y in range(16 * ty, 16 * ty + 16):
                    for x in range(16 * tx, 16 * tx + 16):
                        cin[y, x] = rng.choice(pool, 8, replace=False)
    got = _gpu_propagate(S, n, cin, W, H, jump, 17, 77, 4)
    ref = orc.propagate(S, n, cin, W, H, jump, 17, 77, 4)
    pix = np.arange(W * H)
    u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 17, 77, 4, pix)
    assert compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt) <= 2


def test_propagate_schedule_from_empty_matches_oracle_each_pass(orc):
    """The warm-up schedule from an all-sentinel map: every pass compared with the
    oracle on the oracle's previous output (shared input), then recall."""
    W, H, n = 96, 80, 400
    S = synth.random_sites(n, W, H, 6)
    cur = synth.empty_map(W, H)
    sched = sad.jump_schedule(W, H, 24)
    assert sched == orc.jump_schedule(W, H, 24)
    pix = np.arange(W * H)
    total_bad = 0
    for t, k in enumerate(sched):
        got = _gpu_propagate(S, n, cur, W, H, k, t, 4, 4)
        ref = orc.propagate(S, n, cur, W, H, k, t, 4, 4)
        u, cnt = orc.union_pixels(S, n, cur, W, H, k, t, 4, 4, pix)
        total_bad += compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt)
        cur = ref
    assert total_bad <= 10
    ex = orc.topk_exact(S, n, W, H)
    recall = np.mean([set(a) == set(b) for a, b in zip(cur.reshape(-1, 8), ex.reshape(-1, 8))])
    print(f"exact-list fraction after {len(sched)} passes: {recall:.4f}")
    assert recall > 0.99


@pytest.mark.parametrize("W,H", [(65535, 2), (2, 65535)])
def test_maximum_image_dimension(orc, W, H):
    """Images as wide or as tall as the ABI allows (SAD_MAX_DIM): propagation at the
    first jump of the schedule (32768) and at jump 1, then the fused forward and
    backward (whose image must equal the standalone forward's)."""
    n = 2000
    print(f"maximum dimension W={W} H={H} n={n}", flush=True)
    S, cin = _case(W, H, n, seed=21)
    sched = sad.jump_schedule(W, H, 4)
    assert sched[0] == 32768
    pix = np.arange(W * H)
    for jump, m in ((sched[0], 8), (1, 4)):
        got = _gpu_propagate(S, n, cin, W, H, jump, 7, 31, m)
        ref = orc.propagate(S, n, cin, W, H, jump, 7, 31, m)
        u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 7, 31, m, pix)
        assert compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt) <= max(2, W * H // 2000)
    cand = orc.propagate(S, n, cin, W, H, 1, 0, 1, 4)
    tgt = orc.hard_render(synth.random_sites(n, W, H, 22), n, W, H) + synth.pixel_noise(W, H, 23)
    got, loss = _bwd(S, n, cand, tgt, W, H)
    ref, rloss = orc.render_bwd(S, n, cand, tgt, W, H)
    _check_grads(got, ref)
    assert loss == pytest.approx(rloss, rel=1e-4)


def test_site_records_encode_the_score(orc):
    """The record reproduces the oracle's score: d = s*sqrt((U.delta)^2 +
    (V x delta)^2) - s*r evaluated in float64 from the GPU record vs the oracle's
    float32 score; it carries tau = exp(log tau), the colour, u, e^{+-a} and
    1/|dir|; inactive slots keep x < 0."""
    W, H, n = 90, 70, 500
    S = synth.random_sites(n, W, H, 21)
    S[synth.DX] *= 3.0
    S[synth.DX, 7] = 0.0
    S[synth.DY, 7] = 0.0
    S[synth.X, 9] = -1.0
    g = _rec(S, n).cpu().numpy().astype(np.float64)
    assert g[9, 0] < 0
    S64 = S.astype(np.float64)
    act = np.arange(n) != 9
    assert np.allclose(g[act, 7], np.exp(S64[synth.LOGTAU, act]), rtol=2e-6)
    assert np.array_equal(g[:, 8:11], S64[synth.CR:synth.CB + 1, :n].T)
    nrm = np.hypot(S64[synth.DX], S64[synth.DY])
    ok = nrm > 0
    assert np.allclose(g[ok, 11], 1 / nrm[ok], rtol=1e-6) and g[7, 11] == 0 and g[7, 12] == 1 and g[7, 13] == 0
    assert np.allclose(g[ok, 12], S64[synth.DX, ok] / nrm[ok], atol=1e-6)
    assert np.allclose(g[:, 14], np.exp(S64[synth.A, :n]), rtol=2e-6)
    assert np.allclose(g[:, 14] * g[:, 15], 1.0, rtol=4e-6)
    rng = np.random.default_rng(0)
    pix = rng.integers(0, W * H, 4000)
    ids = rng.integers(0, n, 4000)
    ids[ids == 9] = 8
    ex = (pix % W) + 0.5 - g[ids, 0]
    ey = (pix // W) + 0.5 - g[ids, 1]
    t1 = g[ids, 3] * ex + g[ids, 4] * ey
    t2 = g[ids, 5] * ey - g[ids, 6] * ex
    s = 1.0 / max(W, H)
    d = s * np.sqrt(t1 * t1 + t2 * t2) - s * g[ids, 2]
    ref = orc.score_pairs(S, n, W, H, pix, ids)
    assert np.abs(d - ref).max() < 1e-6


@pytest.mark.parametrize("W,H,n", [(64, 64, 256), (77, 45, 300), (1, 1, 3), (50, 30, 5), (40, 40, 3000)])
def test_topk_exact_matches_oracle(orc, W, H, n):
    print(f"exact W={W} H={H} n={n}", flush=True)
    S = synth.random_sites(n, W, H, 8)
    S[synth.X, ::7] = -1.0
    g = _rec(S, n)
    out = sad.new_map(W, H, g.device)
    sad.topk_exact(g, n, out, W, H)
    torch.cuda.synchronize()
    got = map_to_host(out)
    ref = orc.topk_exact(S, n, W, H)
    pix = np.arange(W * H)
    assert compare_lists(orc, S, n, W, H, pix, got, ref) <= max(1, W * H // 2000)


def _fwd(S, n, cand, W, H):
    R_d = _rec(S, n)
    c = to_dev(cand)
    out = torch.empty((H, W, 3), dtype=torch.float32, device=R_d.device)
    sad.render_fwd_rec(R_d, n, c, W, H, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("W,H,n", SHAPES)
def test_render_fwd_matches_oracle(orc, W, H, n):
    S, cin = _case(W, H, n, seed=2)
    cand = orc.propagate(S, n, cin, W, H, 1, 0, 1, 4)
    got = _fwd(S, n, cand, W, H)
    ref = orc.render_fwd(S, n, cand, W, H)
    assert np.abs(got - ref).max() <= FWD_TOL


def test_render_fwd_edge_inputs(orc):
    W, H, n = 37, 29, 50
    S = synth.random_sites(n, W, H, 9)
    S[synth.X, 3] = -1.0
    S[synth.CR, 4] = np.nan
    S[synth.LOGTAU, 5] = 12.0  # a very sharp site
    S[synth.LOGTAU, 6] = -30.0  # an almost flat one
    cand = synth.random_map(W, H, n + 3, seed=10, p_invalid=0.3, p_dup=0.2)
    cand[0, :, :] = NONE  # empty lists render 0
    got = _fwd(S, n, cand, W, H)
    ref = orc.render_fwd(S, n, cand, W, H)
    assert np.abs(got - ref).max() <= FWD_TOL
    assert (got[0] == 0).all()


def _bwd(S, n, cand, tgt, W, H, grad0=None):
    R_d = _rec(S, n)
    c = to_dev(cand)
    t = to_dev(tgt)
    g = sad.new_grad(S.shape[1], R_d.device)
    if grad0 is not None:
        g[:, :11].copy_(torch.from_numpy(grad0).t())
    loss = sad.new_loss(R_d.device)
    rgb = torch.full((H, W, 3), -7.0, dtype=torch.float32, device=R_d.device)
    sad.render_bwd_rec(R_d, n, c, t, W, H, g, loss, out_rgb=rgb)
    torch.cuda.synchronize()
    gh = g.cpu().numpy().astype(np.float64)
    assert (gh[:, 11:] == 0).all(), "unused words of the gradient records were written"
    # the fused forward output equals the standalone forward bit for bit
    assert np.array_equal(rgb.cpu().numpy(), _fwd(S, n, cand, W, H))
    return np.ascontiguousarray(gh[:, :11].T), float(loss.sum().item())


def _check_grads(got, ref, planes=range(11)):
    for j in planes:
        r = rel_l2(got[j], ref[j])
        assert r <= GRAD_TOL, f"plane {j}: rel L2 {r:.3e}"


@pytest.mark.parametrize("W,H,n", SHAPES)
def test_render_bwd_matches_oracle(orc, W, H, n):
    print(f"bwd W={W} H={H} n={n}", flush=True)
    S, cin = _case(W, H, n, seed=3)
    cand = orc.propagate(S, n, cin, W, H, 1, 0, 1, 4)
    tgt = orc.hard_render(synth.random_sites(n, W, H, 33), n, W, H) + synth.pixel_noise(W, H, 5)
    got, loss = _bwd(S, n, cand, tgt, W, H)
    ref, rloss = orc.render_bwd(S, n, cand, tgt, W, H)
    _check_grads(got, ref)
    assert loss == pytest.approx(rloss, rel=1e-4)


def test_render_bwd_hash_overflow_path(orc):
    """Many tiny sites: a 16x16 tile touches far more than 256 distinct sites, so
    most entries miss the LDS table and go to global atomics."""
    W, H, n = 64, 48, 20000
    S = synth.random_sites(n, W, H, 11)
    cand = synth.random_map(W, H, n, seed=12, p_invalid=0.0, p_dup=0.0)
    tgt = synth.pixel_noise(W, H, 6, 0.3) + 0.5
    got, loss = _bwd(S, n, cand, tgt, W, H)
    ref, rloss = orc.render_bwd(S, n, cand, tgt, W, H)
    _check_grads(got, ref)
    assert loss == pytest.approx(rloss, rel=1e-4)


def test_render_bwd_edge_inputs_and_accumulation(orc):
    W, H, n = 35, 19, 80
    S = synth.random_sites(n, W, H, 13)
    S[synth.X, 2] = -1.0
    S[synth.CG, 3] = np.inf
    S[synth.DX, 4] = 0.0
    S[synth.DY, 4] = 0.0  # degenerate direction
    S[synth.X, 5] = 10.5
    S[synth.Y, 5] = 7.5  # sits exactly on a pixel centre (q = 0 there)
    cand = synth.random_map(W, H, n + 2, seed=14, p_invalid=0.25, p_dup=0.1)
    cand[3, :, :] = NONE
    cand[7, 10, :] = [5, NONE, NONE, NONE, NONE, NONE, NONE, NONE]  # a sole contributor
    tgt = synth.pixel_noise(W, H, 7, 0.3) + 0.5
    g0 = np.random.default_rng(0).normal(0, 1, (11, n)).astype(np.float32)
    got, loss = _bwd(S, n, cand, tgt, W, H, grad0=g0)
    ref, rloss = orc.render_bwd(S, n, cand, tgt, W, H, grad=g0.astype(np.float64))
    _check_grads(got, ref)
    assert np.isfinite(got).all()
    assert loss == pytest.approx(rloss, rel=1e-4)


def _adam_gpu(S, m, v, G, n, step, P, W, H, cfg):
    """G: planes [11][stride]; the library takes per-site records [stride][16]."""
    S_d, m_d, v_d = (to_dev(np.ascontiguousarray(a, dtype=np.float32)) for a in (S, m, v))
    rec = np.zeros((S.shape[1], 16), dtype=np.float32)
    rec[:, :11] = G.T
    rec[:, 11:] = 7.0  # unused words: must survive untouched
    g_d = to_dev(rec)
    rec = sad.new_records(S.shape[1], S_d.device)
    sad.adam_step_rec(S_d, m_d, v_d, g_d, n, step, P, W, H, cfg, rec=rec)
    torch.cuda.synchronize()
    # the refreshed records equal a fresh derivation from the updated sites
    fresh = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, fresh)
    torch.cuda.synchronize()
    assert torch.equal(rec[:n], fresh[:n])
    gh = g_d.cpu().numpy()
    assert (gh[:, 11:] == 7.0).all()
    return [t.cpu().numpy().astype(np.float64) for t in (S_d, m_d, v_d)] + [np.ascontiguousarray(gh[:, :11].T).astype(np.float64)]


@pytest.mark.parametrize("step", [1, 2, 10, 1000])
def test_adam_matches_oracle(orc, step):
    W, H, n, cap = 100, 80, 700, 777  # n_slots < stride; slots beyond n untouched
    S = synth.random_sites(n, W, H, 15, cap)
    S[synth.X, 10] = -1.0
    S[synth.X, 11] = 0.01  # any update this step moves it below 0: clamped
    rng = np.random.default_rng(step)
    m = (rng.normal(0, 1e-3, (10, cap))).astype(np.float32)
    v = (rng.random((10, cap)) * 1e-5).astype(np.float32)
    G = (rng.normal(0, 50, (11, cap))).astype(np.float32)
    G[0, 11] = 1e6  # pushes x below 0: clamped
    G[3, 12] = np.nan
    cfg = sad.AdamConfig()
    got = _adam_gpu(S, m, v, G, n, step, W * H, W, H, cfg)
    p64, m64, v64, g64 = (a.astype(np.float64) for a in (S, m, v, G))
    # the library receives float32 hyper-parameters (sad_adam_cfg); the oracle gets
    # the same float32 values (1 - 0.999f is not 1 - 0.999)
    f32 = lambda x: float(np.float32(x))
    orc.adam_step(p64, m64, v64, g64, n, step, W * H, np.array(cfg.lr, dtype=np.float32).astype(np.float64),
                  f32(cfg.beta1), f32(cfg.beta2), f32(cfg.eps), W, H)
    for a, b in zip(got, (p64, m64, v64, g64)):
        assert np.allclose(a, b, rtol=1e-5, atol=1e-7)
    assert np.array_equal(got[0][:, n:], S[:, n:].astype(np.float64))
    assert got[0][0, 11] == 0.0


def test_empty_image_and_no_sites_are_noops():
    z = torch.zeros((10, 4), dtype=torch.float32, device="cuda")
    m0 = sad.new_map(0, 0)
    sad.topk_propagate_rec(sad.new_records(4), 4, m0, sad.new_map(0, 0), 0, 0, 1, 0, 0, 4)
    out = torch.empty((0, 0, 3), dtype=torch.float32, device="cuda")
    sad.render_fwd_rec(sad.new_records(4), 4, m0, 0, 0, out)
    g = sad.new_grad(4)
    sad.adam_step_rec(z, torch.zeros_like(z), torch.zeros_like(z), g, 0, 1, 1, 1, 1)
    torch.cuda.synchronize()


def test_fitter_iterations_reduce_loss(orc):
    """A short fit: the loss after 60 iterations is below the loss after the first."""
    W, H, n = 96, 64, 600
    S = synth.random_sites(n, W, H, synth.SEED_MODEL)
    tgt = orc.hard_render(synth.random_sites(n, W, H, synth.SEED_TARGET_SITES), n, W, H) + synth.pixel_noise(W, H)
    f = sad.Fitter(to_dev(S), n, to_dev(tgt), W, H)
    assert torch.equal(f.rec[:n], _rec(S, n)[:n])
    losses = []
    for _ in range(60):
        f.loss.zero_()
        f.step()
        losses.append(f.loss.sum().item())
    assert losses[-1] < 0.7 * losses[0]
    assert np.isfinite(losses).all()
