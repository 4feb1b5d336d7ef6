"""GPU parity of the budget-control statistics (sad_densify_stats) against the
oracle, and a fit that splits and prunes between iterations."""
import numpy as np
import pytest
import torch

import soft_voronoi_render_amd as sad
import synth
from sadtest import GRAD_TOL, rel_l2, to_dev

pytestmark = pytest.mark.gpu

PAD = 7.0  # pre-filled value: stats accumulate, and column 7 / rows >= n stay untouched


def _gpu_stats(S, n, cand, tgt, W, H):
    S_d = to_dev(S)
    rec = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, rec)
    st = torch.full((S.shape[1], sad.STAT_LD), PAD, dtype=torch.float32, device=S_d.device)
    sad.densify_stats(rec, n, to_dev(cand), to_dev(tgt), W, H, st)
    torch.cuda.synchronize()
    return st.cpu().numpy().astype(np.float64)


def _check(got, ref, n):
    assert np.all(got[:, 7] == PAD)
    assert np.all(got[n:] == PAD)
    for a in range(7):
        r = rel_l2(got[:n, a] - PAD, ref[:n, a])
        assert r <= GRAD_TOL, f"stat {a}: rel L2 {r:.3e}"


@pytest.mark.parametrize("W,H,n", [(64, 64, 256), (77, 45, 300), (1, 1, 3), (33, 1, 20), (130, 70, 2000)])
def test_densify_stats_match_oracle(orc, W, H, n):
    print(f"densify_stats W={W} H={H} n={n}", flush=True)
    S = synth.random_sites(n, W, H, 21, n + 5)
    S[synth.X, n // 3] = -1.0          # inactive site still listed
    cand = synth.local_map(S, n, W, H, seed=22, radius=6.0)
    tgt = (synth.pixel_noise(W, H, 23, 0.2) + 0.5).astype(np.float32)
    got = _gpu_stats(S, n, cand, tgt, W, H)
    ref = orc.densify_stats(S, n, cand, tgt, W, H)
    _check(got, ref, n)


def test_densify_stats_edge_lists(orc):
    """Sentinels, duplicates, IDs beyond n_slots and the overflow path (more
    distinct sites in a tile than its table holds)."""
    W, H, n = 64, 48, 20000
    S = synth.random_sites(n, W, H, 31)
    cand = synth.random_map(W, H, n, seed=32)
    tgt = (synth.pixel_noise(W, H, 33, 0.3) + 0.5).astype(np.float32)
    got = _gpu_stats(S, n, cand, tgt, W, H)
    ref = orc.densify_stats(S, n, cand, tgt, W, H)
    _check(got, ref, n)


def test_densify_stats_full_size(orc):
    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    print("densify_stats kodak768", flush=True)
    S = synth.random_sites(n, W, H, 41, wl.capacity)
    cand = synth.local_map(S, n, W, H, seed=42, radius=8.0)
    tgt = (synth.pixel_noise(W, H, 43, 0.2) + 0.5).astype(np.float32)
    got = _gpu_stats(S, n, cand, tgt, W, H)
    ref = orc.densify_stats(S, n, cand, tgt, W, H)
    _check(got, ref, n)


def test_fit_with_budget_control(orc):
    """Densify/prune every 40 iterations of a fit: the site count moves by the
    splits minus reused slots, the records match the new sites, pruned sites are
    parked at (-1, -1), and the loss keeps falling."""
    W, H, n, cap = 96, 64, 400, 600
    S = synth.random_sites(n, W, H, synth.SEED_MODEL, cap)
    tgt = orc.hard_render(synth.random_sites(900, W, H, synth.SEED_TARGET_SITES), 900, W, H) + \
        synth.pixel_noise(W, H)
    f = sad.Fitter(to_dev(S), n, to_dev(tgt), W, H)
    losses = []
    cfg = sad.BudgetConfig(split_frac=0.1, prune_frac=0.03)
    for it in range(121):
        f.loss.zero_()
        f.step()
        losses.append(f.loss.sum().item())
        if it in (40, 80):
            before = f.n_slots
            active_before = int((f.sites[0, :before] >= 0).sum())
            ns, npr = f.densify(cfg)
            # counts are floor(fraction * A) with the float32 fraction the C struct holds
            f32 = lambda x: float(np.float32(x))
            assert ns == int(f32(0.1) * active_before) and npr == int(f32(0.03) * active_before)
            assert f.n_slots == before + max(0, ns - npr - (before - active_before))
            assert int((f.sites[0, :f.n_slots] >= 0).sum()) == active_before + ns - npr
            fresh = sad.new_records(cap, f.sites.device)
            sad.site_records(f.sites, f.n_slots, fresh)
            torch.cuda.synchronize()
            assert torch.equal(f.rec[:f.n_slots], fresh[:f.n_slots])
            assert torch.all(f.grad[:, 10] == 0)
    assert np.isfinite(losses).all()
    assert np.mean(losses[-10:]) < 0.95 * np.mean(losses[30:40])
