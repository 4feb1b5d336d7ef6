"""GPU parity of the 16-byte evaluation format and the random-access query
(paperlayer.ai summary, Appendix B.2 "Packed storage for evaluation"; 69574.cn
article, section 5; the summary's abstract on fast random access) through the C
ABI, against the oracle.

* sad_eval_encode: header and every code bit-exact; the only tolerated difference
  is a direction code one apart where the float64 angle sits within 1e-9 of a
  rounding tie (atan2 is not correctly rounded on either side);
* sad_eval_decode: positions, colours, log tau, r and a bit-exact; the direction
  within 3e-7;
* sad_eval_query: colours within 1e-5 of the oracle's float64 blend of its own
  decoded sites, at uniform, border, outside and non-finite points, per-pixel and
  downscaled maps, and at kodak768 with a million points (sampled).
"""
import numpy as np
import pytest
import torch

import oracle
import soft_voronoi_render_amd as sad
import synth
from sadtest import FWD_TOL, to_dev

pytestmark = pytest.mark.gpu


def _edge_sites(n, W, H, seed):
    S = synth.random_sites(n, W, H, seed, n + 5)
    rng = np.random.default_rng(seed)
    S[synth.DX, :n] *= rng.uniform(0.01, 50.0, n)
    if n >= 20:
        S[synth.X, 2] = -1.0                       # inactive
        S[synth.X, 3] = float(W)                   # on the border
        S[synth.Y, 3] = float(H)
        S[synth.CR, 4] = 1.7                       # clamps
        S[synth.CG, 4] = -0.3
        S[synth.CB, 5] = np.nan
        S[synth.LOGTAU, 6] = np.nan                # excluded from the range, codes 0
        S[synth.R, 7] = np.inf
        S[synth.DX, 8] = S[synth.DY, 8] = 0.0      # degenerate direction
        S[synth.DX, 9], S[synth.DY, 9] = -1.0, 0.0  # angle pi folds to 0
        S[synth.DX, 10], S[synth.DY, 10] = 0.0, -1.0
        S[synth.A, 11] = 70000.0                   # a overflows binary16
        S[synth.X, 12] = 0.0
    return S


def _gpu_encode(S, n, W, H):
    S_d = to_dev(S)
    words, hdr = sad.new_eval(S.shape[1], S_d.device)
    words.fill_(-1)
    sad.eval_encode(S_d, n, W, H, words, hdr)
    torch.cuda.synchronize()
    return words, hdr


def _angle_near_tie(S, n):
    dx, dy = S[synth.DX, :n].astype(np.float64), S[synth.DY, :n].astype(np.float64)
    th = np.arctan2(dy, dx)
    th = np.where(th < 0, th + np.pi, th)
    t = th * (65536 / np.pi)
    return np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-9


@pytest.mark.parametrize("W,H,n", [(64, 64, 256), (768, 512, 5000), (1, 1, 3), (4096, 2160, 3000)])
def test_eval_encode_bit_exact(W, H, n):
    print(f"eval encode W={W} H={H} n={n}", flush=True)
    S = _edge_sites(n, W, H, 111)
    words, hdr = _gpu_encode(S, n, W, H)
    got = words.cpu().numpy().view(np.uint32)[:n]
    ref, rh = oracle.eval_encode(S, n, W, H)
    assert np.array_equal(hdr.cpu().numpy().view(np.uint32), rh.view(np.uint32))
    assert np.array_equal(got[:, :3], ref[:, :3])
    assert np.array_equal(got[:, 3] >> 16, ref[:, 3] >> 16)
    da = (got[:, 3].astype(np.int64) & 0xFFFF) - (ref[:, 3].astype(np.int64) & 0xFFFF)
    da = (da + 32768) % 65536 - 32768
    tie = _angle_near_tie(S, n)
    assert np.all((da == 0) | (tie & (np.abs(da) == 1)))
    assert (words[n:] == -1).all()


def test_eval_encode_no_active_sites():
    W, H, n = 16, 16, 4
    S = synth.random_sites(n, W, H, 112)
    S[synth.X, :n] = -1.0
    words, hdr = _gpu_encode(S, n, W, H)
    assert hdr.cpu().tolist() == [0.0, 0.0, 0.0, 0.0]
    assert (words[:n, 0].cpu().numpy().view(np.uint32) == 1 << 31).all() and (words[:n, 1:] == 0).all()


@pytest.mark.parametrize("W,H,n", [(64, 64, 256), (768, 512, 5000)])
def test_eval_decode_matches_oracle(W, H, n):
    S = _edge_sites(n, W, H, 113)
    words, hdr = _gpu_encode(S, n, W, H)
    out = torch.full((10, n + 5), 9.0, dtype=torch.float32, device=words.device)
    sad.eval_decode(words, hdr, n, W, H, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rw, rh = oracle.eval_encode(S, n, W, H)
    ref = oracle.eval_decode(rw, rh, n, W, H)
    for f in (synth.X, synth.Y, synth.LOGTAU, synth.R, synth.CR, synth.CG, synth.CB, synth.A):
        assert np.array_equal(got[f, :n], ref[f].astype(np.float32), equal_nan=True), f
    for f in (synth.DX, synth.DY):
        assert np.abs(got[f, :n] - ref[f]).max() <= 3e-7, f
    assert (got[:, n:] == 9.0).all()


def _query_case(W, H, n, cell, seed):
    S = synth.random_sites(n, W, H, seed)
    rw, rh = oracle.eval_encode(S, n, W, H)
    D = oracle.eval_decode(rw, rh, n, W, H)
    return S, D


@pytest.mark.parametrize("W,H,n,cell", [(64, 64, 256, 1), (77, 45, 300, 3), (130, 70, 2000, 1), (5, 3, 6, 2)])
def test_eval_query_matches_oracle(orc, W, H, n, cell):
    print(f"eval query W={W} H={H} n={n} cell={cell}", flush=True)
    S, D = _query_case(W, H, n, cell, 114)
    cand = orc.topk_exact(D.astype(np.float32), n, W, H, cell=cell)
    rng = np.random.default_rng(115)
    pts = np.concatenate([rng.uniform([0, 0], [W, H], (4000, 2)),
                          [[0.0, 0.0], [W, H], [-5.0, 2.0], [W + 10.0, -3.0], [W - 1e-4, H - 1e-4],
                           [np.nan, 1.0], [1.0, np.inf]]]).astype(np.float32)
    words, hdr = _gpu_encode(S, n, W, H)
    p_d = to_dev(pts)
    out = torch.empty((pts.shape[0], 3), dtype=torch.float32, device=p_d.device)
    sad.eval_query(words, hdr, n, to_dev(cand), W, H, p_d, out, cell=cell)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = orc.query_points(D, n, cand, W, H, pts, cell=cell)
    assert np.abs(got - ref).max() <= FWD_TOL
    assert (got[-2:] == 0).all()


def test_eval_query_full_size_kodak768(orc):
    wl = synth.WORKLOADS["kodak768"]
    W, H, n = wl.W, wl.H, wl.n_sites
    S, D = _query_case(W, H, n, 1, 116)
    cand = orc.topk_exact(D.astype(np.float32), n, W, H)
    words, hdr = _gpu_encode(S, n, W, H)
    rng = np.random.default_rng(117)
    pts = rng.uniform([0, 0], [W, H], (1 << 20, 2)).astype(np.float32)
    p_d = to_dev(pts)
    out = torch.empty((pts.shape[0], 3), dtype=torch.float32, device=p_d.device)
    c_d = to_dev(cand)
    sad.eval_query(words, hdr, n, c_d, W, H, p_d, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        sad.eval_query(words, hdr, n, c_d, W, H, p_d, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(f"kodak768 eval query: {pts.shape[0]} random points in {ms * 1e3:.1f} us "
          f"({pts.shape[0] / ms / 1e3:.0f} Mqueries/s)", flush=True)
    sample = np.unique(rng.choice(pts.shape[0], 20000, replace=False))
    ref = orc.query_points(D, n, cand, W, H, pts[sample])
    assert np.abs(out.cpu().numpy()[sample] - ref).max() <= FWD_TOL
