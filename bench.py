#!/usr/bin/env python3
"""Throughput of the SAD hot path on one MI355X.

One step = one fit iteration over the whole image: one propagation pass of the
candidate map (sad_topk_propagate), the render forward and backward (one
sad_render_bwd launch that writes the rendered image and accumulates the
gradients through the per-tile reduction) and Adam (sad_adam_step), K = 8.  The
standalone forward (sad_render_fwd, the inference render) is timed beside it.  Default workload: the Kodak-shaped fit, 768x512 RGB
float32, N = 50,000 sites, 4 injected candidates per pixel, cold start with the
coarse-to-fine jump schedule 512, 256, ..., 1, 1, ...  Inputs are synthetic and
seeded (sites: uniform positions, colours U[0,1]^3, r U[0,2] px, a N(0,0.5),
direction U[0,pi), log tau U[2,5]; target: hard render of a second seeded site
set plus N(0, 0.01) noise).

Other workloads (`--workload img2048`, `div2k2040`, `edit4096`, `tiny64`) run the
same loop on their shapes; img2048 uses its own recipe (a seeded photo-like image
of polygons and plane waves, gradient-weighted initial sites coloured from it).

The K timed steps replay one HIP graph holding the K iterations (the launches of
a step depend only on the step index, so the whole fit is captured once); the
state is reset to the cold start before the timed replay.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# VALU lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one
# operation per lane per cycle; packed FP32 is not used)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
KERNEL_SRC = os.path.join(ROOT, "soft_voronoi_render_amd", "csrc", "sad_kernels.hip")
# kernel symbol of each timed launch (as rocprofv3 names it)
KERNEL_SYMBOL = {"propagate": "k_propagate<1,256,0>", "fwd_bwd": "k_render_bwd", "adam": "k_adam",
                 "fwd": "k_render_fwd"}


def source_digest():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _profile_rows(path, tag):
    """(source digest, {kernel: fields}) of the `tag kernel=... k=v ...` lines of a
    committed profile summary."""
    rows, digest = {}, None
    if os.path.exists(path):
        for line in open(path):
            line = line.strip()
            if line.startswith("source_sha256:"):
                digest = line.split(":", 1)[1].strip()
            elif line.startswith(tag + " "):
                kv = dict(f.split("=", 1) for f in line.split()[1:])
                rows[kv["kernel"]] = kv
    return digest, rows


def measured_valu_issue(workload, kernel):
    """Fraction of the VALU issue cycles a launch uses (SQ_INSTS_VALU x 4 cycles over
    1024 SIMDs x duration x 2.4 GHz) from the committed counter summary, or None when
    there is none or the kernel source has changed since."""
    digest, rows = _profile_rows(os.path.join(ROOT, "profiles", f"valu_issue_{workload}.txt"), "valu")
    if digest != source_digest() or KERNEL_SYMBOL[kernel] not in rows:
        return None
    return float(rows[KERNEL_SYMBOL[kernel]]["issue_frac"])


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the same counters on a plain copy of
    known size), or None when there is none for this kernel and workload or the
    kernel source has changed since the counters were taken."""
    digest, rows = _profile_rows(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt"), "traffic")
    if digest != source_digest() or KERNEL_SYMBOL[kernel] not in rows:
        return None
    return float(rows[KERNEL_SYMBOL[kernel]]["bytes_per_launch"])


def algorithmic_ops(P, N, M, K=8):
    """VALU lane operations per launch that the literal algorithm needs (an FMA,
    compare or select counts one; a square root, exp or reciprocal counts one).

    propagate: (5K + M) candidates per pixel (own list, 4 neighbour lists,
               injected IDs), each scored (12: delta 2, metric projections 4,
               quadratic form 3, sqrt 1, d = s q - s r 2) and offered to the
               sorted top-K (18: key 3, compare 1, amortised insertion 14) = 30
    fwd_bwd:   per entry 20 for the forward (score 12, logit 1, max 1, exp 2,
               normaliser 1, colour 3) and 60 for the backward (gamma 7, colour
               gradient 3, log tau 1, d 1, position 12, r 1, a 4, direction 8,
               removal delta 12, 11 accumulations) = 80, plus 10 per pixel
               (residual, loss, 1/Z)
    fwd:       per entry 20 (as above) plus 4 per pixel
    adam:      12 per parameter, 10 parameters per site
    """
    return {
        "propagate": P * (5 * K + M) * 30,
        "fwd_bwd": P * (K * 80 + 10),
        "adam": N * 10 * 12,
        "fwd": P * (K * 20 + 4),
    }


def algorithmic_bytes(P, N):
    """Compulsory HBM bytes per launch (each tensor byte read once, written once).

    propagate: map in + map out (64 B/px) + the 32-byte scoring half of each
               site record (32 B/site)
    fwd_bwd:   map (32 B/px) + target (12 B/px) + image out (12 B/px) + the site
               record (64 B/site) + one read-modify-write flush of the 11
               accumulators (88 B/site)
    adam:      params, m, v read and written (240 B/site) + the 10 gradients of
               the site's record read and zeroed (80 B/site) + the site record
               written (64 B/site)
    fwd:       (standalone render, not part of the step) map (32 B/px) + image
               out (12 B/px) + the 44 bytes of the record the blend reads
    """
    return {
        "propagate": 64 * P + 32 * N,
        "fwd_bwd": 56 * P + 152 * N,
        "adam": 384 * N,
        "fwd": 44 * P + 44 * N,
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def make_inputs(wl, dev):
    import torch

    import soft_voronoi_render_amd as sad
    import synth

    W, H, n = wl.W, wl.H, wl.n_sites
    if wl.name == "img2048":
        # the 2k workload: a seeded photo-like image (polygons and plane waves on
        # mid-grey) and gradient-weighted initial sites coloured from it
        img = synth.polygon_image(W, H, synth.SEED_TARGET_SITES)
        S = synth.gradient_weighted_sites(img, n, synth.SEED_MODEL, wl.capacity)
        return S, torch.from_numpy(np.ascontiguousarray(img, dtype=np.float32)).to(dev)
    S = synth.random_sites(n, W, H, synth.SEED_MODEL, wl.capacity)
    S2 = synth.random_sites(n, W, H, synth.SEED_TARGET_SITES)
    noise = synth.pixel_noise(W, H, synth.SEED_NOISE)
    # target: hard (argmin) render of the second site set = colour of the first
    # entry of its exact top-K map (brute force on the GPU), plus noise
    S2_d = torch.from_numpy(S2).to(dev)
    g2 = sad.new_records(n, dev)
    sad.site_records(S2_d, n, g2)
    ex = sad.new_map(W, H, dev)
    sad.topk_exact(g2, n, ex, W, H)
    first = ex[:, :, 0].long()
    col = S2_d[4:7].t()  # [n][3]
    tgt = torch.where((first >= 0)[..., None], col[first.clamp(min=0)], torch.zeros(1, device=dev))
    tgt = (tgt + torch.from_numpy(noise).to(dev)).contiguous()
    return S, tgt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="kodak768")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of graph replays (for counter collection)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (reference for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SAD hot path here is built and measured on a single "
              "MI355X; sharding by image bands across GPUs is designed but not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    import soft_voronoi_render_amd as sad
    import synth

    sad.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    W, H, N, P = wl.W, wl.H, wl.n_sites, wl.P
    S0, tgt = make_inputs(wl, dev)
    S0_d = torch.from_numpy(S0).to(dev)
    fit = sad.Fitter(S0_d.clone(), N, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT)
    stream = torch.cuda.current_stream()

    def reset():
        fit.sites.copy_(S0_d)
        fit.refresh_records()
        fit.m.zero_()
        fit.v.zero_()
        fit.grad.zero_()
        fit.maps[0].fill_(-1)
        fit.maps[1].fill_(-1)
        fit.cur = 0
        fit.it = 0
        fit.passes = 0
        fit.warm_end = 0
        fit.loss.zero_()

    # warm-up (untimed): the first iterations of the fit
    for _ in range(args.warmup):
        fit.step()
    torch.cuda.synchronize()

    # timed region: K iterations from the cold start
    reset()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                fit.step()
        reset()
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            fit.step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1)
    ms_per_step = ms / args.steps
    value = P * args.steps / (ms * 1e-3) / 1e6

    # quality after the fit: loss of one more iteration
    fit.it = args.steps
    fit.passes = args.steps
    fit.loss.zero_()
    fit.step()
    torch.cuda.synchronize()
    mse = fit.loss.sum().item() / (3 * P)
    psnr = 10 * np.log10(1.0 / max(mse, 1e-30))
    # recall of the maintained map against the exact top-K (brute force on the GPU)
    ex = sad.new_map(W, H, dev)
    sad.topk_exact(fit.rec, N, ex, W, H)
    cur = fit.cand
    a, _ = torch.sort(cur.view(-1, 8), dim=1)
    b, _ = torch.sort(ex.view(-1, 8), dim=1)
    exact_frac = (a == b).all(dim=1).float().mean().item()

    # per-kernel average launch duration: R back-to-back launches of each kernel
    # on the fitted state, one graph replay bracketed by events on this stream
    kb = algorithmic_bytes(P, N)
    kdur = {}
    R = args.kernel_reps
    launches = {
        "propagate": lambda i: sad.topk_propagate(fit.rec, N, fit.maps[i % 2], fit.maps[1 - i % 2], W, H, 1,
                                                  1000 + i, synth.SEED_INJECT, wl.n_inject),
        "fwd_bwd": lambda i: sad.render_bwd(fit.rec, N, fit.cand, fit.target, W, H, fit.grad, fit.loss, fit.rgb),
        "adam": lambda i: sad.adam_step(fit.sites, fit.m, fit.v, fit.grad, N, 500 + i, P, W, H, fit.adam, fit.rec),
        "fwd": lambda i: sad.render_fwd(fit.rec, N, fit.cand, W, H, fit.rgb),
    }
    for name, fn in launches.items():
        g = None
        if not args.no_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(R):
                    fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if g is not None:
            g.replay()
        else:
            for i in range(R):
                fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        kdur[name] = e0.elapsed_time(e1) / R * 1e-3  # s per launch
    if args.copy_calibration_mib > 0:
        # a plain elementwise copy kernel: reads and writes exactly `nbytes`
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    step_kernels = ("propagate", "fwd_bwd", "adam")
    dominant = max(step_kernels, key=kdur.get)
    kops = algorithmic_ops(P, N, wl.n_inject)
    kernels = {k: {"us": round(kdur[k] * 1e6, 3), "GBps": round(kb[k] / kdur[k] / 1e9, 1),
                   "hbm_frac": round(kb[k] / kdur[k] / 1e9 / HBM_PEAK_GBS, 4),
                   "Tops": round(kops[k] / kdur[k] / 1e12, 2),
                   "alu_frac": round(kops[k] / kdur[k] / 1e12 / VALU_PEAK_TOPS, 4),
                   "valu_issue_frac": measured_valu_issue(wl.name, k)} for k in kdur}
    # the bound of a kernel: the roof its algorithmic work reaches first
    alu_bound = kernels[dominant]["alu_frac"] >= kernels[dominant]["hbm_frac"]
    if alu_bound:
        roofline = {"bound": "alu", "kernel": dominant, "achieved": kernels[dominant]["Tops"],
                    "peak": round(VALU_PEAK_TOPS, 2), "unit": "T VALU lane-ops/s",
                    "frac": kernels[dominant]["alu_frac"], "algorithmic_ops_per_launch": kops[dominant]}
    else:
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": kernels[dominant]["GBps"],
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dominant]["hbm_frac"]}
    roofline.update({"traffic": measured_traffic(wl.name, dominant), "algorithmic_bytes_per_launch": kb[dominant],
                     "hbm_frac": kernels[dominant]["hbm_frac"],
                     "valu_issue_frac": measured_valu_issue(wl.name, dominant)})

    out = {
        "metric": "Mpixel-iters/s (propagate+fwd+bwd+Adam, K=8) and % of HBM peak",
        "value": round(value, 2),
        "unit": "Mpixel-iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "W": W, "H": H, "n_sites": N, "K": 8, "n_inject": wl.n_inject,
            "schedule": "cold start, jumps B/2..1 then 1", "graph": graph is not None,
            "hbm_frac_whole_step": round(sum(kb[k] for k in step_kernels) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                         4),
            "psnr_db_after": round(float(psnr), 3), "exact_top8_fraction_after": round(exact_frac, 4),
            "kernels": kernels,
        },
        "roofline": roofline,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, S0, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, S0, budget_s):
    """The oracle's own iteration (propagate, forward, backward, Adam) on the same
    sites, timed on the host cores, for as many iterations as fit the budget."""
    import oracle
    import synth

    oracle.build(force=False)
    # the host's share of cores: OMP_NUM_THREADS where the environment sets it
    cores = min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1))
    oracle.set_threads(cores)
    cores = oracle.get_threads()
    W, H, N, P = wl.W, wl.H, wl.n_sites, wl.P
    S = S0.copy()
    tgt = (synth.pixel_noise(W, H, 99, 0.25) + 0.5).astype(np.float32)
    cand = synth.empty_map(W, H)
    params = S.astype(np.float64)
    m = np.zeros((10, S.shape[1]))
    v = np.zeros((10, S.shape[1]))
    grad = np.zeros((11, S.shape[1]))
    lr = np.array([0.1, 0.1, 0.02, 0.05, 0.01, 0.01, 0.01, 0.02, 0.02, 0.02])
    sched = oracle.jump_schedule(W, H, 10_000)
    it, t_used = 0, 0.0
    while t_used < budget_s and it < 10_000:
        t0 = time.perf_counter()
        S32 = params.astype(np.float32)
        cand = oracle.propagate(S32, N, cand, W, H, sched[it], it, synth.SEED_INJECT, wl.n_inject)
        oracle.render_fwd(params, N, cand, W, H)
        oracle.render_bwd(params, N, cand, tgt, W, H, grad=grad)
        oracle.adam_step(params, m, v, grad, N, it + 1, P, lr, 0.9, 0.999, 1e-8, W, H)
        t_used += time.perf_counter() - t0
        it += 1
    return {"value": round(P * it / t_used / 1e6, 4), "unit": "Mpixel-iters/s", "cores": cores, "kind": "oracle",
            "sample": f"first {it} iterations of the {wl.name} fit ({W}x{H}, N={N}), same sites; target replaced "
                      f"by seeded noise (the oracle's cost does not depend on target values); {t_used:.1f} s",
            "cpu": cpu_model()}


if __name__ == "__main__":
    main()
