"""Pins of the oracle's 16-byte evaluation format and random-access query
(paperlayer.ai summary, Appendix B.2 "Packed storage for evaluation"; 69574.cn
article, section 5: 15-bit coordinates, 11/11/10-bit colour, 16-bit temperature,
radius and direction angle, float16 anisotropy).

* words of hand-picked sites worked out by hand here: round-to-even ties in the
  position, colour, log tau and r codes, the per-image ranges, the angle folding
  (dir and -dir give one code; pi folds to 0), a degenerate direction, an inactive
  slot;
* encode -> decode errors stay within half a quantisation step per field;
* the decoded blend at pixel centres is the render of the decoded sites, bit for
  bit; at arbitrary points it equals a float64 numpy blend written out here from
  the explicit metric matrix.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _site(S, i, x, y, lt, r, rgb, d, a):
    S[:, i] = [x, y, lt, r, rgb[0], rgb[1], rgb[2], d[0], d[1], a]


def test_eval_words_worked_by_hand():
    W, H = 1024, 512  # 32767/1024 and 32767/512 are exact in float32
    S = synth.empty_sites(6)
    _site(S, 0, 512.0, 256.0, 2.0, 0.0, (0.5, 1.0, 0.25), (1.0, 1.0), 0.1)
    _site(S, 1, 100.0, 0.0, 5.0, 2.0, (0.0, 0.0, 1.0), (0.0, 1.0), 0.0)
    _site(S, 2, 1024.0, 512.0, 3.5, 1.0, (1.5, -0.2, 0.5), (-1.0, 0.0), -2.0)
    _site(S, 3, 0.0, 511.0, 2.0, 0.5, (0.1, 0.2, 0.3), (0.0, -1.0), 1.0)
    _site(S, 4, 7.0, 7.0, 9.0, 9.0, (0.1, 0.2, 0.3), (0.0, 0.0), 0.0)   # degenerate direction
    S[:, 5] = [-1.0, 3.0, 99.0, 99.0, 1, 1, 1, 1, 0, 0]                 # inactive: ignored by the ranges
    w, hdr = oracle.eval_encode(S, 5, W, H)
    # ranges over the active slots: log tau in [2, 9], r in [0, 9]
    assert hdr.tolist() == [2.0, np.float32(7.0) / np.float32(65535), 0.0, np.float32(9.0) / np.float32(65535)]
    # site 0: x 512 * 31.9990234375 = 16383.5 -> even 16384; y 256 * 63.998046875 = 16383.5 -> 16384
    #         R 0.5 * 2047 = 1023.5 -> 1024; G 1 -> 2047; B 0.25 * 1023 = 255.75 -> 256
    #         log tau 2 (the minimum) -> 0; r 0 -> 0; dir (1,1): 45 degrees -> 16384; a 0.1 -> 0x2e66
    assert w[0].tolist() == [16384 | 16384 << 15, 1024 | 2047 << 11 | 256 << 22, 0, 16384 | 0x2E66 << 16]
    # site 1: x 3199.90234375 -> 3200; y 0; colour (0, 0, 1023); log tau 5: 3 * (65535/7) = 28086.43 -> 28086;
    #         r 2: 2 * (65535/9) = 14563.33 -> 14563; dir (0, 1): 90 degrees -> 32768; a 0
    inv_lt = np.float32(65535) / np.float32(7)
    inv_r = np.float32(65535) / np.float32(9)
    assert int(np.rint(np.float32(3) * inv_lt)) == 28086 and int(np.rint(np.float32(2) * inv_r)) == 14563
    assert w[1].tolist() == [3200, 1023 << 22, 28086 | 14563 << 16, 32768]
    # site 2: x = W -> 32767, y = H -> 32767; R 1.5 clamps to 2047, G < 0 clamps to 0, B 0.5 * 1023 = 511.5 -> 512;
    #         dir (-1, 0): atan2 = pi folds to 0; a -2 -> 0xc000
    q_lt2 = int(np.rint(np.float32(1.5) * inv_lt))
    q_r2 = int(np.rint(np.float32(1.0) * inv_r))
    assert w[2].tolist() == [32767 | 32767 << 15, 2047 | 512 << 22, q_lt2 | q_r2 << 16, 0xC000 << 16]
    # site 3: dir (0, -1): -90 degrees folds to +90 -> 32768; a 1.0 -> 0x3c00
    assert w[3, 3] == 32768 | 0x3C00 << 16 and w[3, 0] == 0 | int(np.rint(np.float32(511) * np.float32(63.998046875))) << 15
    # site 4: degenerate direction -> angle code 0; log tau 9 and r 9 are the maxima -> 65535
    assert w[4, 2] == 65535 | 65535 << 16 and w[4, 3] & 0xFFFF == 0
    # an inactive slot is one flag bit
    w6, _ = oracle.eval_encode(S, 6, W, H)
    assert w6[5].tolist() == [1 << 31, 0, 0, 0] and np.array_equal(w6[:5], w)


def test_eval_round_trip_error_bounds():
    W, H, n = 768, 512, 20000
    S = synth.random_sites(n, W, H, 101)
    S[synth.DX, :n] *= np.random.default_rng(102).uniform(0.01, 100, n)  # |dir| does not matter
    w, hdr = oracle.eval_encode(S, n, W, H)
    D = oracle.eval_decode(w, hdr, n, W, H)
    S64 = S.astype(np.float64)
    # half a step, plus the float32 roundings of the encode product and of the decode (a few ulp of W)
    assert np.abs(D[synth.X] - S64[synth.X]).max() <= 0.5 * W / 32767 + 4 * np.spacing(np.float32(W))
    assert np.abs(D[synth.Y] - S64[synth.Y]).max() <= 0.5 * H / 32767 + 4 * np.spacing(np.float32(H))
    assert np.abs(D[synth.X] - S64[synth.X]).max() > 0.45 * W / 32767  # and it is not finer than that
    for f, q in ((synth.CR, 2047), (synth.CG, 2047), (synth.CB, 1023)):
        assert np.abs(D[f] - S64[f]).max() <= 0.5 / q + 4 * np.spacing(np.float32(1))
    for f, k in ((synth.LOGTAU, 1), (synth.R, 3)):
        assert np.abs(D[f] - S64[f]).max() <= 0.5 * float(hdr[k]) * (1 + 1e-3) + 1e-6
    th = np.arctan2(S64[synth.DY], S64[synth.DX])
    th_hat = np.arctan2(D[synth.DY], D[synth.DX])
    err = np.abs(((th - th_hat) + np.pi / 2) % np.pi - np.pi / 2)  # axis angle, mod pi
    assert err.max() <= 0.5 * np.pi / 65536 + 4 * np.spacing(np.float32(np.pi))  # the decode's float32 product
    assert np.array_equal(D[synth.A].astype(np.float32), S[synth.A].astype(np.float16).astype(np.float32))


def test_query_at_centres_is_the_render(orc):
    W, H, n = 60, 44, 400
    S = synth.random_sites(n, W, H, 103)
    w, hdr = oracle.eval_encode(S, n, W, H)
    D = oracle.eval_decode(w, hdr, n, W, H)
    for cell in (1, 3):
        cand = orc.topk_exact(D.astype(np.float32), n, W, H, cell=cell)
        rows, cols = np.divmod(np.arange(W * H), W)
        pts = np.stack([cols + 0.5, rows + 0.5], -1).astype(np.float32)
        q = orc.query_points(D, n, cand, W, H, pts, cell=cell)
        img = orc.render_fwd(D, n, cand, W, H, cell=cell)
        assert np.array_equal(q, img.reshape(-1, 3))


def _blend_numpy(D, lst, X, Y, W, H):
    s = 1.0 / max(W, H)
    l, col = [], []
    for i in lst:
        if i == 0xFFFFFFFF or D[synth.X, i] < 0:
            continue
        u = np.array([D[synth.DX, i], D[synth.DY, i]])
        u = u / np.linalg.norm(u)
        v = np.array([-u[1], u[0]])
        a = D[synth.A, i]
        G = math.exp(a) * np.outer(u, u) + math.exp(-a) * np.outer(v, v)
        dlt = np.array([X - D[synth.X, i], Y - D[synth.Y, i]])
        d = s * math.sqrt(dlt @ G @ dlt) - s * D[synth.R, i]
        l.append(-math.exp(D[synth.LOGTAU, i]) * d)
        col.append(D[synth.CR:synth.CB + 1, i])
    if not l:
        return np.zeros(3)
    l = np.array(l)
    e = np.exp(l - l.max())
    return (e[:, None] * np.array(col)).sum(0) / e.sum()


def test_query_at_points_matches_explicit_blend(orc):
    W, H, n = 50, 30, 200
    S = synth.random_sites(n, W, H, 104)
    w, hdr = oracle.eval_encode(S, n, W, H)
    D = oracle.eval_decode(w, hdr, n, W, H)
    cand = orc.topk_exact(D.astype(np.float32), n, W, H, cell=2)
    rng = np.random.default_rng(105)
    pts = np.concatenate([rng.uniform([0, 0], [W, H], (300, 2)),
                          [[-3.0, 5.0], [W + 4.0, H + 1.0], [0.0, 0.0], [W - 1e-3, H - 1e-3]]]).astype(np.float32)
    q = orc.query_points(D, n, cand, W, H, pts, cell=2)
    for p, (X, Y) in enumerate(pts.astype(np.float64)):
        col = min(max(int(math.floor(X)), 0), W - 1)
        row = min(max(int(math.floor(Y)), 0), H - 1)
        ref = _blend_numpy(D, cand[row // 2, col // 2], X, Y, W, H)
        assert np.abs(q[p] - ref).max() < 1e-12, p
    bad = orc.query_points(D, n, cand, W, H, np.array([[np.nan, 1.0], [1.0, np.inf]], dtype=np.float32), cell=2)
    assert (bad == 0).all()
