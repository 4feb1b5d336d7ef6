"""GPU parity of the jump-flood prepass (sad_jfa_seed, sad_jfa_pass) against the
oracle, through the C ABI: candidate sets identical except where scores differ by
less than the selection tolerance, lists sentinel-padded and ascending."""
import numpy as np
import pytest
import torch

import soft_voronoi_render_amd as sad
import synth
from sadtest import compare_lists, map_to_host, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(64, 64, 256), (77, 45, 300), (1, 1, 3), (33, 1, 20), (1, 50, 40), (130, 70, 2000)]


def _rec(S, n):
    S_d = to_dev(S)
    g = sad.new_records(S.shape[1], S_d.device)
    sad.site_records(S_d, n, g)
    return g


def _edge_sites(n, W, H, seed):
    S = synth.random_sites(n, W, H, seed)
    if n >= 20:
        S[synth.X, :6] = min(W - 1, 3) + np.linspace(0.05, 0.95, 6)  # six sites in one pixel
        S[synth.Y, :6] = min(H - 1, 2) + np.linspace(0.95, 0.05, 6)
        S[synth.X, 10] = -1.0
        S[synth.X, 11] = np.nan
        S[synth.Y, 12] = np.inf
        S[synth.X, 13] = float(W)
        S[synth.Y, 14] = -5.0
        S[synth.X, 15] = 1e6
    return S


@pytest.mark.parametrize("W,H,n", SHAPES)
def test_jfa_seed_matches_oracle(orc, W, H, n):
    print(f"jfa seed W={W} H={H} n={n}", flush=True)
    S = _edge_sites(n, W, H, 61)
    g = _rec(S, n)
    c = sad.new_map(W, H, g.device)
    c.fill_(7)  # the seed pass writes the whole map
    sad.jfa_seed(g, n, c, W, H)
    torch.cuda.synchronize()
    got = map_to_host(c)
    ref = orc.jfa_seed(S, n, W, H)
    assert (got[..., 4:] == 0xFFFFFFFF).all()
    pix = np.arange(W * H, dtype=np.uint32)
    bad = compare_lists(orc, S, n, W, H, pix, got.reshape(-1, 8), ref.reshape(-1, 8))
    assert bad <= max(1, W * H // 5000)


@pytest.mark.parametrize("W,H,n", SHAPES)
@pytest.mark.parametrize("step", [1, 2, 5, 8, 16, 64, 1000])
def test_jfa_pass_matches_oracle(orc, W, H, n, step):
    print(f"jfa pass W={W} H={H} n={n} step={step}", flush=True)
    S = _edge_sites(n, W, H, 62)
    cin = synth.random_map(W, H, n + 3, seed=63)
    g = _rec(S, n)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device)
    sad.jfa_pass(g, n, a, b, W, H, step)
    torch.cuda.synchronize()
    got = map_to_host(b).reshape(-1, 8)
    ref = orc.jfa_pass(S, n, cin, W, H, step).reshape(-1, 8)
    assert (got[:, 4:] == 0xFFFFFFFF).all()
    pix = np.arange(W * H, dtype=np.uint32)
    u, cnt = orc.jfa_union_pixels(S, n, cin, W, H, step, pix)
    bad = compare_lists(orc, S, n, W, H, pix, got, ref, u, cnt)
    assert bad <= max(2, W * H // 2000)


def test_jfa_prepass_kodak768_each_pass(orc):
    """The full prepass at the Kodak-shaped size, each pass on the oracle's previous
    output, whole image compared."""
    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    S = synth.random_sites(n, W, H, synth.SEED_MODEL)
    g = _rec(S, n)
    c = sad.new_map(W, H, g.device)
    sad.jfa_seed(g, n, c, W, H)
    torch.cuda.synchronize()
    cur = orc.jfa_seed(S, n, W, H)
    pix = np.arange(W * H, dtype=np.uint32)
    total_bad = compare_lists(orc, S, n, W, H, pix, map_to_host(c).reshape(-1, 8), cur.reshape(-1, 8))
    for k in sad.jfa_steps(W, H):
        print(f"jfa pass step {k}", flush=True)
        a = to_dev(cur)
        b = sad.new_map(W, H, a.device)
        sad.jfa_pass(g, n, a, b, W, H, k)
        torch.cuda.synchronize()
        got = map_to_host(b).reshape(-1, 8)
        ref = orc.jfa_pass(S, n, cur, W, H, k)
        mism = np.nonzero([set(x) != set(y) for x, y in zip(got, ref.reshape(-1, 8))])[0]
        if mism.size:
            u, cnt = orc.jfa_union_pixels(S, n, cur, W, H, k, pix[mism])
            total_bad += compare_lists(orc, S, n, W, H, pix[mism], got[mism], ref.reshape(-1, 8)[mism], u, cnt)
        cur = ref
    assert total_bad <= 50


def test_jfa_then_propagation_recall(orc):
    """Prepass (seed + 10 flood passes) and 4 propagation passes at jump 1 against
    the regular cold start (jumps 512 .. 1, then 4 at 1): recall of both against
    the exact top-8 on sampled pixels, reported; the prepass route must reach a
    comparable map."""
    wl = synth.WORKLOADS["kodak768"]
    W, H, n, M = wl.W, wl.H, wl.n_sites, wl.n_inject
    S = synth.random_sites(n, W, H, synth.SEED_MODEL)
    g = _rec(S, n)
    a = sad.new_map(W, H, g.device)
    b = sad.new_map(W, H, g.device)
    res = sad.jfa_prepass(g, n, a, b, W, H)
    other = b if res.data_ptr() == a.data_ptr() else a
    for t in range(4):
        sad.topk_propagate_rec(g, n, res, other, W, H, 1, t, synth.SEED_INJECT, M)
        res, other = other, res
    jfa_map = map_to_host(res).reshape(-1, 8).copy()
    c = sad.new_map(W, H, g.device)
    d = sad.new_map(W, H, g.device)
    for t, k in enumerate(sad.jump_schedule(W, H, 14)):
        sad.topk_propagate_rec(g, n, c, d, W, H, k, t, synth.SEED_INJECT, M)
        c, d = d, c
    torch.cuda.synchronize()
    reg_map = map_to_host(c).reshape(-1, 8)
    rng = np.random.default_rng(768)
    pix = np.unique(rng.choice(W * H, 3000, replace=False)).astype(np.uint32)
    ref = orc.topk_exact_pixels(S, n, W, H, pix)
    rec_jfa = np.mean([len(set(x) & set(y)) / 8 for x, y in zip(jfa_map[pix], ref)])
    rec_reg = np.mean([len(set(x) & set(y)) / 8 for x, y in zip(reg_map[pix], ref)])
    ex_jfa = np.mean([set(x) == set(y) for x, y in zip(jfa_map[pix], ref)])
    ex_reg = np.mean([set(x) == set(y) for x, y in zip(reg_map[pix], ref)])
    print(f"kodak768 recall per entry / exact sets: prepass+4 {rec_jfa:.4f} / {ex_jfa:.4f}, "
          f"cold-start schedule (14 passes) {rec_reg:.4f} / {ex_reg:.4f}", flush=True)
    assert rec_jfa > 0.9 and rec_jfa >= rec_reg - 0.05
