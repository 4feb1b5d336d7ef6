"""The two larger workload runs, on the GPU through the C ABI:

* edit4096 (4096x4096, 1M sites, 8 injected per pixel): converge the map, move a
  seeded 10% of the sites by up to 256 px, refresh it with one coarse-to-fine
  schedule (jumps 2048 .. 1), then render forward and backward.  The refreshed map
  is measured against the plain definition -- the oracle's brute-force exact top-8
  -- on 4096 seeded pixels (recall; the pages report most pixels exact after a
  dozen rounds, with their own N unstated).
* div2k2040 (2040x1356, 200k sites, capacity 220k): a fit with budget control
  every 50 iterations; the site count stays within the +-10% the workload allows,
  records stay consistent and the loss falls.

Both are properties at full size, not element-wise parity (which the per-pass
tests cover): the oracle is too slow to follow a million-site map through dozens
of passes.
"""
import time

import numpy as np
import pytest
import torch

import bench
import soft_voronoi_render_amd as sad
import synth
from sadtest import map_to_host, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _refresh(rec, n, a, b, W, H, jumps, pass0, seed, m, scr=None):
    for t, k in enumerate(jumps):
        sad.topk_propagate_rec(rec, n, a, b, W, H, k, pass0 + t, seed, m, scr=scr)
        a, b = b, a
    return a, b


def test_edit4096_refresh_recall(orc):
    wl = synth.WORKLOADS["edit4096"]
    W, H, n, M = wl.W, wl.H, wl.n_sites, wl.n_inject
    print("edit4096: converge", flush=True)
    S = synth.random_sites(n, W, H, synth.SEED_MODEL)
    S_d = to_dev(S)
    rec = sad.new_records(n, S_d.device)
    sad.site_records(S_d, n, rec)
    a = sad.new_map(W, H, S_d.device)
    b = sad.new_map(W, H, S_d.device)
    sched = sad.jump_schedule(W, H, 12)
    assert sched[0] == 2048 and sched[11] == 1
    a, b = _refresh(rec, n, a, b, W, H, sched + sched + [1] * 20, 0, synth.SEED_INJECT, M)
    # the edit
    S2 = synth.displace_sites(S, n, W, H, seed=77)
    S2_d = to_dev(S2)
    sad.site_records(S2_d, n, rec)
    scr = sad.new_screen(n, S2_d.device)  # propagation screens candidates, as the fit does
    sad.site_screen(S2_d, n, W, H, scr)
    torch.cuda.synchronize()
    print("edit4096: refresh", flush=True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    a, b = _refresh(rec, n, a, b, W, H, sched, 1000, synth.SEED_INJECT, M, scr)
    e1.record()
    tgt = (synth.pixel_noise(W, H, 5, 0.2) + 0.5).astype(np.float32)
    t_d = to_dev(tgt)
    rgb = torch.empty((H, W, 3), dtype=torch.float32, device=S_d.device)
    g = sad.new_grad(n, S_d.device)
    loss = sad.new_loss(S_d.device)
    e2 = torch.cuda.Event(enable_timing=True)
    e2.record()
    sad.render_bwd_rec(rec, n, a, t_d, W, H, g, loss, rgb)
    e3 = torch.cuda.Event(enable_timing=True)
    e3.record()
    torch.cuda.synchronize()
    refresh_ms, fb_ms = e0.elapsed_time(e1), e2.elapsed_time(e3)
    assert np.isfinite(loss.sum().item())
    rng = np.random.default_rng(4096)
    pix = np.unique(rng.choice(W * H, 4096, replace=False)).astype(np.uint32)
    pix_d = torch.from_numpy(pix.astype(np.int64)).to(a.device)
    got = map_to_host(a.view(-1, 8)[pix_d])
    # the other route after a large edit: rebuild with the jump-flood prepass (seed
    # pass + 12 flood passes keeping four), then 4 propagation passes at jump 1
    print("edit4096: jump-flood reinitialisation", flush=True)
    e4 = torch.cuda.Event(enable_timing=True)
    e5 = torch.cuda.Event(enable_timing=True)
    e4.record()
    res = sad.jfa_prepass(rec, n, b, a, W, H)
    oth = a if res.data_ptr() == b.data_ptr() else b
    for t in range(4):
        sad.topk_propagate_rec(rec, n, res, oth, W, H, 1, 2000 + t, synth.SEED_INJECT, M, scr=scr)
        res, oth = oth, res
    e5.record()
    torch.cuda.synchronize()
    jfa_ms = e4.elapsed_time(e5)
    got_jfa = map_to_host(res.view(-1, 8)[pix_d])
    print("edit4096: oracle exact top-8 on 4096 pixels", flush=True)
    t0 = time.time()
    ref = orc.topk_exact_pixels(S2, n, W, H, pix)
    exact = np.mean([set(x) == set(y) for x, y in zip(got, ref)])
    per_entry = np.mean([len(set(x) & set(y)) / 8.0 for x, y in zip(got, ref)])
    exact_j = np.mean([set(x) == set(y) for x, y in zip(got_jfa, ref)])
    per_entry_j = np.mean([len(set(x) & set(y)) / 8.0 for x, y in zip(got_jfa, ref)])
    print(f"edit4096: refresh {refresh_ms:.2f} ms (12 passes), fused fwd+bwd {fb_ms:.2f} ms, "
          f"exact-set recall {exact:.4f}, per-entry recall {per_entry:.4f} (oracle {time.time() - t0:.1f} s)",
          flush=True)
    print(f"edit4096: jump-flood reinit + 4 passes {jfa_ms:.2f} ms, exact-set recall {exact_j:.4f}, "
          f"per-entry recall {per_entry_j:.4f}", flush=True)
    assert per_entry > 0.9 and exact > 0.6
    assert per_entry_j > 0.9


def test_div2k2040_fit_with_budget_control():
    wl = synth.WORKLOADS["div2k2040"]
    W, H, n, cap = wl.W, wl.H, wl.n_sites, wl.capacity
    # the benchmark's inputs: seeded sites, and as target the hard render of a second
    # seeded site set (the exact nearest site of every pixel) plus noise
    S, tgt = bench.make_inputs(wl, torch.device("cuda:0"))
    f = sad.Fitter(to_dev(S), n, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT)
    losses, counts = [], []
    t0 = time.time()
    for it in range(wl.iters):
        f.loss.zero_()
        f.step()
        if it % 10 == 9:
            losses.append(f.loss.sum().item())
        if it % 50 == 49 and it < wl.iters - 1:
            torch.cuda.synchronize()
            td = time.time()
            ns, npr = f.densify()
            torch.cuda.synchronize()
            td = time.time() - td
            active = int((f.sites[0, :f.n_slots] >= 0).sum())
            counts.append(active)
            assert f.n_slots <= cap
            assert abs(active - n) <= 0.1 * n, "budget control moved N beyond +-10%"
            print(f"div2k2040 it {it + 1}: split {ns}, pruned {npr}, active {active}, slots {f.n_slots}, "
                  f"budget control {td * 1e3:.1f} ms", flush=True)
    torch.cuda.synchronize()
    print(f"div2k2040: {wl.iters} iterations with budget control in {time.time() - t0:.1f} s", flush=True)
    fresh = sad.new_records(cap, f.sites.device)
    sad.site_records(f.sites, f.n_slots, fresh)
    torch.cuda.synchronize()
    assert torch.equal(f.rec[:f.n_slots], fresh[:f.n_slots])
    assert np.isfinite(losses).all()
    assert losses[-1] < 0.8 * losses[2]
    assert len(counts) == 5


def test_kodak768_refresh_frequency():
    """Candidate-field refresh every 1, 8 and 16 iterations (the summary's B.3
    reports 8-16 iterations between updates leave the final PSNR unchanged): PSNR
    of the 200-iteration kodak768 fit and time per iteration, reported; the
    infrequent schedules must stay close in PSNR and be faster.  The warm-up runs
    one pass per iteration here, the schedule these bounds were set on."""
    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    S, tgt = bench.make_inputs(wl, torch.device("cuda:0"))
    res = {}
    for every, passes in ((1, 1), (8, 1), (16, 1), (8, 2)):
        f = sad.Fitter(to_dev(S), n, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT,
                       refresh_every=every, passes_per_refresh=passes, warmup="interleaved")
        for _ in range(3):  # warm the kernels up
            f.step()
        f = sad.Fitter(to_dev(S), n, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT,
                       refresh_every=every, passes_per_refresh=passes, warmup="interleaved")
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
        res[(every, passes)] = (psnr, e0.elapsed_time(e1) / wl.iters)
        print(f"kodak768 refresh every {every} x {passes} pass: PSNR {psnr:.3f} dB, "
              f"{res[(every, passes)][1] * 1e3:.1f} us per iteration", flush=True)
    base_psnr, base_t = res[(1, 1)]
    for key in ((8, 1), (16, 1)):
        assert res[key][1] < base_t
        assert res[key][0] > base_psnr - 0.5
