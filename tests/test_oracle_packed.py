"""Pins of the packed candidate-site buffer's oracle (paperlayer.ai summary,
Appendix B.2 "Packed candidate sites": 16 bytes per site, float16 pairs of
position, (log tau, r), direction and (a, 0)).

* the words of a site whose fields are chosen binary16 cases -- exact values,
  round-to-nearest-even ties, the largest finite value, overflow, the smallest
  subnormal -- equal the bit patterns IEEE 754 fixes for them, in the stated
  order and halves, and an inactive slot packs x = -1;
* rounding stays within half an ulp (2^-11 relative) in the normal range, which
  truncation would break;
* sites already representable in binary16 are unchanged by the rounding, so their
  packed-mode selection equals the float32 selection;
* the packed-mode exact top-8 equals a brute-force float64 top-8 computed from the
  words decoded independently here (numpy's float16 view), up to near-ties.
"""
import numpy as np
import pytest

import oracle
import synth

NONE = 0xFFFFFFFF


def test_pack_words_bit_patterns():
    S = synth.empty_sites(3)
    S[:, 0] = [1.0, 0.5, -2.0, 2049.0, 0.3, 0.3, 0.3, 65504.0, 2.0 ** -24, 0.1]
    S[:, 1] = [2051.0, 65520.0, 1e6, 3 * 2.0 ** -25, 0.3, 0.3, 0.3, -0.0, 1.0, 0.0]
    S[:, 2] = [-1e-8, 7.0, 0.0, 1.0, 0.3, 0.3, 0.3, 1.0, 0.0, np.nan]
    w = oracle.pack_words(S, 3)
    # x=1.0 (0x3c00), y=0.5 (0x3800); log tau=-2 (0xc000), r=2049 -> tie, even: 2048 (0x6800)
    # dir_x=65504 (largest finite, 0x7bff), dir_y=2^-24 (smallest subnormal, 0x0001); a=0.1 (0x2e66)
    assert w[0].tolist() == [0x3C00 | 0x3800 << 16, 0xC000 | 0x6800 << 16, 0x7BFF | 0x0001 << 16, 0x2E66]
    # x=2051 -> tie, even: 2052 (0x6802); y=65520 overflows to +inf (0x7c00); log tau=1e6 -> inf;
    # r=3*2^-25 -> tie between 2^-24 and 2^-23, even: 2^-23 (0x0002); dir_x=-0 (0x8000); a=0
    assert w[1].tolist() == [0x6802 | 0x7C00 << 16, 0x7C00 | 0x0002 << 16, 0x8000 | 0x3C00 << 16, 0x0000]
    # an inactive slot (x < 0, however small) packs x = -1 (0xbc00); a = NaN stays NaN
    assert w[2, 0] & 0xFFFF == 0xBC00 and w[2, 0] >> 16 == 0x4700
    assert (w[2, 3] & 0x7C00) == 0x7C00 and (w[2, 3] & 0x03FF) != 0 and w[2, 3] >> 16 == 0


def test_rounding_is_nearest():
    rng = np.random.default_rng(1)
    v = (rng.uniform(-1, 1, 200_000) * 10.0 ** rng.uniform(-4, 4.5, 200_000)).astype(np.float32)
    S = synth.empty_sites(v.size)
    S[synth.LOGTAU] = v
    S[synth.X] = 1.0
    back = oracle.rounded_sites(S, v.size)[synth.LOGTAU].astype(np.float64)
    normal = np.abs(v) >= 2.0 ** -14
    err = np.abs(back[normal] - v[normal].astype(np.float64)) / np.abs(v[normal].astype(np.float64))
    assert err.max() <= 2.0 ** -11 * (1 + 1e-12)
    assert err.max() > 2.0 ** -12  # rounding does happen


def test_representable_sites_select_as_float32(orc):
    W, H, n = 90, 70, 600
    S = synth.random_sites(n, W, H, 81)
    # positions on a 1/16 px grid below 128 px, radii on 1/64, the rest on small dyadic sets
    S[synth.X, :n] = np.round(S[synth.X, :n] * 16) / 16
    S[synth.Y, :n] = np.round(S[synth.Y, :n] * 16) / 16
    S[synth.R, :n] = np.round(S[synth.R, :n] * 64) / 64
    S[synth.A, :n] = np.round(S[synth.A, :n] * 256) / 256
    S[synth.DX, :n] = np.round(S[synth.DX, :n] * 1024) / 1024
    S[synth.DY, :n] = np.round(S[synth.DY, :n] * 1024) / 1024
    S[synth.LOGTAU, :n] = np.round(S[synth.LOGTAU, :n] * 256) / 256
    S[synth.X, 5] = -1.0
    T = oracle.rounded_sites(S, n)
    assert np.array_equal(T, S)
    assert np.array_equal(orc.topk_exact(T, n, W, H), orc.topk_exact(S, n, W, H))


def _decoded_scores(words, n, W, H):
    """Scores of every site at every pixel centre, float64, from the words decoded here."""
    h = words.astype(np.uint32)
    lo = lambda w: (w & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    hi = lambda w: (w >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    x, y, r = lo(h[:, 0]), hi(h[:, 0]), hi(h[:, 1])
    dx, dy, a = lo(h[:, 2]), hi(h[:, 2]), lo(h[:, 3])
    nrm = np.hypot(dx, dy)
    ux = np.where(nrm ** 2 >= 1e-30, dx / np.where(nrm > 0, nrm, 1), 1.0)
    uy = np.where(nrm ** 2 >= 1e-30, dy / np.where(nrm > 0, nrm, 1), 0.0)
    rows, cols = np.divmod(np.arange(W * H), W)
    ex = cols[:, None] + 0.5 - x[None, :]
    ey = rows[:, None] + 0.5 - y[None, :]
    al = ux * ex + uy * ey
    be = -uy * ex + ux * ey
    s = 1.0 / max(W, H)
    d = s * np.sqrt(np.exp(a) * al ** 2 + np.exp(-a) * be ** 2) - s * r
    d[:, x < 0] = np.inf
    return d


def test_packed_selection_matches_decoded_brute_force(orc):
    W, H, n = 40, 30, 300
    S = synth.random_sites(n, W, H, 82)
    S[synth.X, :n] *= 30.0  # positions up to ~1200 px: spacing 0.5-1 px in binary16
    S[synth.Y, :n] *= 30.0
    S[synth.X, :n] = np.minimum(S[synth.X, :n], W - 0.01)  # keep a few hundred near the image
    S[synth.Y, :n] = np.minimum(S[synth.Y, :n], H - 0.01)
    S[synth.X, 7] = -1e-8  # inactive, must stay inactive after rounding
    words = oracle.pack_words(S, n)
    got = orc.topk_exact(oracle.rounded_sites(S, n), n, W, H).reshape(-1, 8)
    d = _decoded_scores(words, n, W, H)
    order = np.lexsort((np.broadcast_to(np.arange(n), d.shape), d), axis=1)[:, :8]
    bad = 0
    for p in range(W * H):
        if set(got[p]) != set(order[p]):
            a = np.sort(d[p, got[p]])
            b = np.sort(d[p, order[p]])
            assert np.abs(a - b).max() < 1e-6, p
            bad += 1
    assert bad <= 3
    assert 7 not in got
