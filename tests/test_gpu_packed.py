"""GPU parity of the packed candidate-site buffer (paperlayer.ai summary, Appendix
B.2 "Packed candidate sites") through the C ABI.

* sad_pack_sites writes exactly the oracle's words (IEEE binary16, nearest even),
  edge values included;
* sad_adam_step's packed output equals a fresh packing of the updated sites;
* every selection entry point reading the packed buffer (propagation on the tile
  table and table-free, on per-pixel and downscaled maps; the jump-flood seed and
  flood pass; the exact top-8) matches the oracle's selection on the sites with
  their packed fields rounded to binary16, under the usual candidate-set rule;
* at kodak768 a 200-iteration fit reading the packed buffer is reported next to
  the fit reading the records (time per iteration, PSNR).
"""
import numpy as np
import pytest
import torch

import oracle
import soft_voronoi_render_amd as sad
import synth
from sadtest import NONE, compare_lists, map_to_host, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(64, 64, 256), (77, 45, 300), (300, 70, 2000), (33, 1, 20)]


def _packed(S, n):
    S_d = to_dev(S)
    p = sad.new_packed(S.shape[1], S_d.device)
    sad.pack_sites(S_d, n, p)
    return p


def _sites(n, W, H, seed):
    S = synth.random_sites(n, W, H, seed, n + 3)
    if n >= 20:
        S[synth.X, 3] = -1e-8         # inactive, however small
        S[synth.X, 5] = float(W) + 2
        S[synth.Y, 6] = np.nan
    return S


def test_pack_sites_bit_exact(orc):
    n = 5000
    S = synth.random_sites(n, 4096, 3000, 91, n + 7)
    rng = np.random.default_rng(92)
    S[synth.LOGTAU, :n] = rng.normal(0, 30, n)
    S[synth.R, :n] = rng.uniform(0, 1, n) * 10.0 ** rng.uniform(-9, 6, n)
    S[synth.DX, :n] *= 10.0 ** rng.uniform(-9, 5, n)
    S[:, :6] = [[1.0, 2051.0, -1e-8, 65519.0, 65520.0, 2049.0],
                [0.5, 65520.0, 7.0, 3.0, 1.0, 0.0],
                [-2.0, 1e6, 0.0, 1.0, 2.0, 3.0],
                [2049.0, 3 * 2.0 ** -25, 1.0, 2.0 ** -25, 2.0 ** -26, 1e-30],
                [0.3] * 6, [0.3] * 6, [0.3] * 6,
                [65504.0, -0.0, 1.0, -65520.0, 1.0, 0.0],
                [2.0 ** -24, 1.0, 0.0, 1.0, 0.0, 1.0],
                [0.1, 0.0, np.nan, np.inf, -np.inf, 0.0]]
    got = _packed(S, n).cpu().numpy().view(np.uint32)[:n]
    ref = orc.pack_words(S, n)
    nan_ref = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x03FF) != 0)
    nan_got = ((got & 0x7C00) == 0x7C00) & ((got & 0x03FF) != 0)
    assert np.array_equal(nan_got, nan_ref)
    same = (got == ref) | (nan_ref & nan_got)
    # a NaN may differ in its payload bits only (checked per half-word)
    lo_ok = ((got & 0xFFFF) == (ref & 0xFFFF)) | (_is_nan16(got & 0xFFFF) & _is_nan16(ref & 0xFFFF))
    hi_ok = ((got >> 16) == (ref >> 16)) | (_is_nan16(got >> 16) & _is_nan16(ref >> 16))
    assert (lo_ok & hi_ok).all(), np.argwhere(~(lo_ok & hi_ok))[:5]
    assert same.mean() > 0.999


def _is_nan16(h):
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)


def test_adam_refreshes_packed_words():
    W, H, n, cap = 100, 80, 700, 777
    S = synth.random_sites(n, W, H, 93, cap)
    S[synth.X, 10] = -1.0
    rng = np.random.default_rng(94)
    S_d = to_dev(S)
    m = torch.zeros((10, cap), device=S_d.device)
    v = torch.zeros((10, cap), device=S_d.device)
    g = sad.new_grad(cap, S_d.device)
    g[:, :10] = torch.from_numpy(rng.normal(0, 50, (cap, 10)).astype(np.float32)).to(S_d.device)
    rec = sad.new_records(cap, S_d.device)
    pk = sad.new_packed(cap, S_d.device)
    pk.fill_(-7)
    sad.adam_step_rec(S_d, m, v, g, n, 3, W * H, W, H, rec=rec, packed=pk)
    fresh = sad.new_packed(cap, S_d.device)
    sad.pack_sites(S_d, n, fresh)
    torch.cuda.synchronize()
    assert torch.equal(pk[:n], fresh[:n])
    assert (pk[n:] == -7).all()


@pytest.mark.parametrize("W,H,n", SHAPES)
@pytest.mark.parametrize("jump,m,cell", [(1, 4, 1), (3, 0, 1), (16, 8, 1), (1, 4, 3), (2, 4, 2)])
def test_packed_propagate_matches_oracle(orc, W, H, n, jump, m, cell):
    print(f"packed propagate W={W} H={H} n={n} jump={jump} m={m} cell={cell}", flush=True)
    S = _sites(n, W, H, 95)
    T = oracle.rounded_sites(S, n)
    Hm, Wm, _ = sad.map_shape(W, H, cell)
    cin = synth.random_map(Wm, Hm, n + 3, seed=96)
    pk = _packed(S, n)
    a = to_dev(cin)
    b = sad.new_map(W, H, a.device, cell=cell)
    sad.topk_propagate_rec(pk, n, a, b, W, H, jump, 77, 5, m, cell=cell)
    torch.cuda.synchronize()
    got = map_to_host(b)
    ref = orc.propagate(T, n, cin, W, H, jump, 77, 5, m, cell=cell)
    pix = np.arange(Wm * Hm, dtype=np.uint32)
    u, cnt = orc.union_pixels(T, n, cin, W, H, jump, 77, 5, m, pix, cell=cell)
    assert compare_lists(orc, T, n, W, H, pix, got, ref, u, cnt, cell=cell) <= max(2, pix.size // 2000)
    assert 3 not in got


@pytest.mark.parametrize("W,H,n", SHAPES)
def test_packed_exact_and_jfa_match_oracle(orc, W, H, n):
    print(f"packed exact+jfa W={W} H={H} n={n}", flush=True)
    S = _sites(n, W, H, 97)
    T = oracle.rounded_sites(S, n)
    pk = _packed(S, n)
    pix = np.arange(W * H, dtype=np.uint32)
    ex = sad.new_map(W, H, pk.device)
    sad.topk_exact(pk, n, ex, W, H)
    sd = sad.new_map(W, H, pk.device)
    sad.jfa_seed(pk, n, sd, W, H)
    torch.cuda.synchronize()
    assert compare_lists(orc, T, n, W, H, pix, map_to_host(ex), orc.topk_exact(T, n, W, H)) <= max(1, pix.size // 2000)
    seed_ref = orc.jfa_seed(T, n, W, H)
    assert compare_lists(orc, T, n, W, H, pix, map_to_host(sd), seed_ref) <= max(1, pix.size // 2000)
    for k in sad.jfa_steps(W, H)[-2:]:
        x = to_dev(seed_ref)
        y = sad.new_map(W, H, x.device)
        sad.jfa_pass(pk, n, x, y, W, H, k)
        torch.cuda.synchronize()
        ref = orc.jfa_pass(T, n, seed_ref, W, H, k)
        u, cnt = orc.jfa_union_pixels(T, n, seed_ref, W, H, k, pix)
        assert compare_lists(orc, T, n, W, H, pix, map_to_host(y), ref, u, cnt) <= max(2, pix.size // 1000)


def test_packed_propagate_full_size_kodak768(orc):
    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    S = synth.random_sites(n, W, H, 98, wl.capacity)
    T = oracle.rounded_sites(S, n)
    cin = synth.local_map(S, n, W, H, seed=99, radius=8.0)
    pk = _packed(S, n)
    a = to_dev(cin)
    pix = np.unique(np.random.default_rng(7).choice(W * H, 20000, replace=False)).astype(np.uint32)
    for jump in (1, 64):
        print(f"packed propagate kodak768 jump={jump}", flush=True)
        b = sad.new_map(W, H, a.device)
        sad.topk_propagate_rec(pk, n, a, b, W, H, jump, 4242, synth.SEED_INJECT, wl.n_inject)
        torch.cuda.synchronize()
        got = map_to_host(b).reshape(-1, 8)[pix]
        ref = orc.propagate_pixels(T, n, cin, W, H, jump, 4242, synth.SEED_INJECT, wl.n_inject, pix)
        u, cnt = orc.union_pixels(T, n, cin, W, H, jump, 4242, synth.SEED_INJECT, wl.n_inject, pix)
        assert compare_lists(orc, T, n, W, H, pix, got, ref, u, cnt) <= pix.size // 2000


def test_packed_kodak768_fit():
    """The 200-iteration kodak768 fit with the candidate passes on the records and on
    the packed buffer: time per iteration and PSNR, reported; the packed fit must
    converge to within 0.3 dB."""
    import bench

    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    S, tgt = bench.make_inputs(wl, torch.device("cuda:0"))
    res = {}
    for packed in (False, True):
        f = sad.Fitter(to_dev(S), n, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT, packed=packed)
        for _ in range(3):
            f.step()
        f = sad.Fitter(to_dev(S), n, tgt, W, H, n_inject=wl.n_inject, seed=synth.SEED_INJECT, packed=packed)
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
        res[packed] = (psnr, e0.elapsed_time(e1) / wl.iters)
        print(f"kodak768 {'packed' if packed else 'records'}: PSNR {psnr:.3f} dB, {res[packed][1] * 1e3:.1f} us per "
              f"iteration", flush=True)
        if packed:
            fresh = sad.new_packed(f.sites.shape[1], f.sites.device)
            sad.pack_sites(f.sites, n, fresh)
            torch.cuda.synchronize()
            assert torch.equal(f.packed[:n], fresh[:n])
    assert res[True][0] > res[False][0] - 0.3


@pytest.mark.parametrize("W,H,n,cell", [(130, 70, 2000, 2), (77, 45, 300, 4)])
def test_packed_grid_exact_and_jfa(orc, W, H, n, cell):
    """The packed buffer on a downscaled map: exact top-8 and the jump-flood seed and
    last flood passes against the oracle on the rounded sites and the same grid."""
    print(f"packed grid W={W} H={H} n={n} cell={cell}", flush=True)
    S = _sites(n, W, H, 99)
    T = oracle.rounded_sites(S, n)
    pk = _packed(S, n)
    Hm, Wm, _ = sad.map_shape(W, H, cell)
    pix = np.arange(Wm * Hm, dtype=np.uint32)
    ex = sad.new_map(W, H, pk.device, cell=cell)
    sad.topk_exact(pk, n, ex, W, H, cell=cell)
    sd = sad.new_map(W, H, pk.device, cell=cell)
    sad.jfa_seed(pk, n, sd, W, H, cell=cell)
    torch.cuda.synchronize()
    assert compare_lists(orc, T, n, W, H, pix, map_to_host(ex), orc.topk_exact(T, n, W, H, cell=cell),
                         cell=cell) <= 1
    seed_ref = orc.jfa_seed(T, n, W, H, cell=cell)
    assert compare_lists(orc, T, n, W, H, pix, map_to_host(sd), seed_ref, cell=cell) <= 1
    for k in sad.jfa_steps(W, H, cell=cell)[-2:]:
        x = to_dev(seed_ref)
        y = sad.new_map(W, H, x.device, cell=cell)
        sad.jfa_pass(pk, n, x, y, W, H, k, cell=cell)
        torch.cuda.synchronize()
        ref = orc.jfa_pass(T, n, seed_ref, W, H, k, cell=cell)
        u, cnt = orc.jfa_union_pixels(T, n, seed_ref, W, H, k, pix, cell=cell)
        assert compare_lists(orc, T, n, W, H, pix, map_to_host(y), ref, u, cnt, cell=cell) <= 2
