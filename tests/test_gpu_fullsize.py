"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses (the tile-table propagation at jumps up to 8, the five-region
table beyond, the fused forward+backward launch, Adam refreshing the site
records).

The oracle checks full images where it finishes in seconds and sampled pixels
otherwise (its per-pixel functions evaluate any subset of pixels exactly).
Inputs are synthetic: seeded sites of each workload's size, spatially coherent
random candidate lists (synth.local_map) and a noise target -- the parity of a
kernel does not depend on what the target image shows.
"""
import numpy as np
import pytest
import torch

import soft_voronoi_render_amd as sad
import synth
from sadtest import FWD_TOL, GRAD_TOL, compare_lists, map_to_host, rel_l2, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

SAMPLE = 20_000


def _setup(name, seed=1):
    wl = synth.WORKLOADS[name]
    W, H, n = wl.W, wl.H, wl.n_sites
    S = synth.random_sites(n, W, H, seed, wl.capacity)
    cin = synth.local_map(S, n, W, H, seed=seed + 7, radius=8.0)
    return wl, S, cin


def _sample(W, H, seed=3, k=SAMPLE):
    rng = np.random.default_rng(seed)
    pix = rng.choice(W * H, size=min(k, W * H), replace=False).astype(np.uint32)
    # always include the four corners and an edge run
    extra = np.array([0, W - 1, (H - 1) * W, W * H - 1] + list(range(min(W, 40))), dtype=np.uint32)
    return np.unique(np.concatenate([pix, extra]))


@pytest.mark.parametrize("name", ["kodak768", "img2048", "div2k2040", "edit4096"])
@pytest.mark.parametrize("jump", [1, 4, 64])
def test_propagate_full_size_sampled(orc, name, jump):
    wl, S, cin = _setup(name)
    W, H, n = wl.W, wl.H, wl.n_sites
    print(f"propagate {name} jump={jump}", flush=True)
    S_d = to_dev(S)
    rec = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, rec)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device)
    sad.topk_propagate_rec(rec, n, a, b, W, H, jump, 4242, synth.SEED_INJECT, wl.n_inject)
    torch.cuda.synchronize()
    got = map_to_host(b).reshape(-1, 8)
    del a, b
    pix = _sample(W, H)
    ref = orc.propagate_pixels(S, n, cin, W, H, jump, 4242, synth.SEED_INJECT, wl.n_inject, pix)
    u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 4242, synth.SEED_INJECT, wl.n_inject, pix)
    bad = compare_lists(orc, S, n, W, H, pix, got[pix], ref, u, cnt)
    assert bad <= max(2, pix.size // 2000)


@pytest.mark.parametrize("name", ["kodak768", "img2048", "div2k2040", "edit4096"])
def test_fused_forward_backward_full_size(orc, name):
    """The launch a fit step uses: image (sampled vs the oracle's forward) and all
    11 gradient planes (the oracle's full backward) plus the loss."""
    wl, S, cin = _setup(name, seed=2)
    W, H, n = wl.W, wl.H, wl.n_sites
    print(f"fwd+bwd {name}", flush=True)
    # the map the kernels read: the oracle's own propagation of the coherent lists
    cand = orc.propagate(S, n, cin, W, H, 1, 7, synth.SEED_INJECT, wl.n_inject)
    tgt = (synth.pixel_noise(W, H, 11, 0.2) + 0.5).astype(np.float32)
    S_d = to_dev(S)
    rec = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, rec)
    c_d = to_dev(cand)
    t_d = to_dev(tgt)
    g_d = sad.new_grad(S.shape[1], S_d.device)
    loss = sad.new_loss(S_d.device)
    rgb = torch.empty((H, W, 3), dtype=torch.float32, device=S_d.device)
    sad.render_bwd_rec(rec, n, c_d, t_d, W, H, g_d, loss, rgb)
    torch.cuda.synchronize()
    got_rgb = rgb.cpu().numpy().reshape(-1, 3)
    got_g = sad.grad_planes(g_d).cpu().numpy().astype(np.float64)
    got_loss = loss.sum().item()
    del c_d, t_d, rgb, g_d
    pix = _sample(W, H)
    ref_rgb = orc.render_fwd_pixels(S, n, cand, W, H, pix)
    assert np.abs(got_rgb[pix] - ref_rgb).max() <= FWD_TOL
    ref_g, ref_loss = orc.render_bwd(S, n, cand, tgt, W, H)
    for j in range(11):
        r = rel_l2(got_g[j], ref_g[j])
        assert r <= GRAD_TOL, f"plane {j}: rel L2 {r:.3e}"
    assert got_loss == pytest.approx(ref_loss, rel=1e-4)


@pytest.mark.parametrize("name", ["kodak768", "edit4096"])
def test_adam_full_size(orc, name):
    wl = synth.WORKLOADS[name]
    W, H, n = wl.W, wl.H, wl.n_sites
    S = synth.random_sites(n, W, H, 5, wl.capacity)
    rng = np.random.default_rng(9)
    G = rng.normal(0, 30, (11, S.shape[1])).astype(np.float32)
    m = (rng.normal(0, 1e-3, (10, S.shape[1]))).astype(np.float32)
    v = (rng.random((10, S.shape[1])) * 1e-5).astype(np.float32)
    S_d, m_d, v_d = to_dev(S), to_dev(m), to_dev(v)
    g_d = sad.new_grad(S.shape[1], S_d.device)
    g_d[:, :11].copy_(torch.from_numpy(G).t())
    rec = sad.new_records(S.shape[1], S_d.device)
    cfg = sad.AdamConfig()
    sad.adam_step_rec(S_d, m_d, v_d, g_d, n, 3, W * H, W, H, cfg, rec=rec)
    torch.cuda.synchronize()
    p64, m64, v64, g64 = (a.astype(np.float64) for a in (S, m, v, G))
    f32 = lambda x: float(np.float32(x))
    orc.adam_step(p64, m64, v64, g64, n, 3, W * H, np.array(cfg.lr, dtype=np.float32).astype(np.float64),
                  f32(cfg.beta1), f32(cfg.beta2), f32(cfg.eps), W, H)
    assert np.allclose(S_d.cpu().numpy(), p64, rtol=1e-5, atol=1e-7)
    assert np.allclose(m_d.cpu().numpy(), m64, rtol=1e-5, atol=1e-9)
    assert np.allclose(v_d.cpu().numpy(), v64, rtol=1e-5, atol=1e-12)
    fresh = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, fresh)
    torch.cuda.synchronize()
    assert torch.equal(rec[:n], fresh[:n])


def test_kodak768_schedule_each_pass(orc):
    """The bench's cold start at full size: the first 12 passes of the coarse-to-fine
    schedule (512 .. 1, then 1), each pass on the oracle's previous output, whole
    image compared."""
    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    S = synth.random_sites(n, W, H, synth.SEED_MODEL)
    S_d = to_dev(S)
    rec = sad.new_records(n, S_d.device)
    sad.site_records(S_d, n, rec)
    cur = synth.empty_map(W, H)
    sched = sad.jump_schedule(W, H, 12)
    pix = np.arange(W * H, dtype=np.uint32)
    total_bad = 0
    for t, k in enumerate(sched):
        print(f"pass {t} jump {k}", flush=True)
        a = to_dev(cur)
        b = sad.new_map(W, H, a.device)
        sad.topk_propagate_rec(rec, n, a, b, W, H, k, t, synth.SEED_INJECT, wl.n_inject)
        torch.cuda.synchronize()
        got = map_to_host(b)
        ref = orc.propagate(S, n, cur, W, H, k, t, synth.SEED_INJECT, wl.n_inject)
        mism = np.nonzero([set(x) != set(y) for x, y in zip(got.reshape(-1, 8), ref.reshape(-1, 8))])[0]
        if mism.size:
            u, cnt = orc.union_pixels(S, n, cur, W, H, k, t, synth.SEED_INJECT, wl.n_inject, pix[mism])
            total_bad += compare_lists(orc, S, n, W, H, pix[mism], got.reshape(-1, 8)[mism],
                                       ref.reshape(-1, 8)[mism], u, cnt)
        cur = ref
    assert total_bad <= 50
