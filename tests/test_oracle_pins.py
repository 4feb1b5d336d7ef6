"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks the oracle against mathematics the pages fix, a closed form,
a textbook/library routine, an invariant, a brute-force recomputation, or a
hand-worked case under tests/golden/.  A plausible slip in the oracle (a dropped
term, a wrong sign or index, a transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth

NONE = 0xFFFFFFFF
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sites(n, W, H, seed, cap=None):
    return synth.random_sites(n, W, H, seed, cap)


def _pix_centres(W, H):
    rows, cols = np.divmod(np.arange(W * H), W)
    return cols + 0.5, rows + 0.5


# ------------------------------------------------------------------ RNG pins
def _gf2_matmul(A, B):
    return (A.astype(np.int64) @ B.astype(np.int64)) % 2


def _gf2_pow(M, e):
    R = np.eye(M.shape[0], dtype=np.int64)
    while e:
        if e & 1:
            R = _gf2_matmul(R, M)
        M = _gf2_matmul(M, M)
        e >>= 1
    return R


def test_xorshift32_is_full_period_linear_map(orc):
    """Marsaglia (2003): xorshift32 with shifts (13,17,5) is a linear map on GF(2)^32
    of multiplicative order 2^32 - 1 (every non-zero state is on one cycle)."""
    rng = np.random.default_rng(0)
    for _ in range(200):
        a, b = (int(x) for x in rng.integers(0, 2**32, 2, dtype=np.uint64))
        assert orc.xorshift32(a ^ b) == orc.xorshift32(a) ^ orc.xorshift32(b)
    T = np.zeros((32, 32), dtype=np.int64)
    for j in range(32):
        y = orc.xorshift32(1 << j)
        for i in range(32):
            T[i, j] = (y >> i) & 1
    order = 2**32 - 1
    I = np.eye(32, dtype=np.int64)
    assert np.array_equal(_gf2_pow(T, order), I)
    for p in (3, 5, 17, 257, 65537):  # 2^32 - 1 = 3*5*17*257*65537
        assert not np.array_equal(_gf2_pow(T, order // p), I)


def test_pcg_hash_is_the_published_permutation(orc):
    """Jarzynski & Olano (JCGT 2020) 'pcg' hash: LCG step (PCG's 32-bit multiplier
    747796405, increment 2891336453) then the RXS-M-XS output permutation
    (multiplier 277803737).  Pinned by inverting each stage from its definition."""
    M1, C1, M2 = 747796405, 2891336453, 277803737
    inv1, inv2 = pow(M1, -1, 2**32), pow(M2, -1, 2**32)

    def invert(out):
        word = out ^ (out >> 22)
        t = (word * inv2) & 0xFFFFFFFF
        sh = (t >> 28) + 4
        state = t
        for _ in range(10):
            state = t ^ (state >> sh)
        return ((state - C1) * inv1) & 0xFFFFFFFF

    rng = np.random.default_rng(1)
    vals = [0, 1, 2, 0xFFFFFFFF, 0x80000000] + [int(x) for x in rng.integers(0, 2**32, 500, dtype=np.uint64)]
    outs = [orc.pcg_hash(v) for v in vals]
    assert [invert(o) for o in outs] == vals
    assert len(set(outs)) == len(outs)


def test_injection_chain_and_range_reduction(orc):
    """Injected IDs = multiply-shift (Lemire 2019) of successive xorshift32 states
    seeded by pcg(pcg(pcg(seed) ^ password) ^ pixel); password = jump<<16 | (pass & 0xffff)
    (paperlayer.ai summary, Appendix B.3 'Jump schedule')."""
    seed, jump, pidx, pix = 1234, 64, 70000, 4097
    assert orc.pass_word(jump, pidx) == (64 << 16) | (70000 & 0xFFFF)
    h = orc.pcg_hash(orc.pcg_hash(orc.pcg_hash(seed) ^ orc.pass_word(jump, pidx)) ^ pix)
    for n_slots in (1, 7, 256, 50_000, 2**20, 2**32 - 1):
        ids = orc.inject_ids(seed, jump, pidx, pix, n_slots, 6)
        x = h
        for j in range(6):
            x = orc.xorshift32(x)
            assert int(ids[j]) == (x * n_slots) >> 32
            assert int(ids[j]) < n_slots
    # power-of-two range: the top bits of the state
    ids = orc.inject_ids(seed, jump, pidx, pix, 256, 4)
    x = h
    for j in range(4):
        x = orc.xorshift32(x)
        assert int(ids[j]) == x >> 24
    # only the low 16 bits of the pass index enter the pass word
    assert np.array_equal(orc.inject_ids(seed, jump, 5, pix, 1000, 8), orc.inject_ids(seed, jump, 5 + 65536, pix, 1000, 8))
    assert not np.array_equal(orc.inject_ids(seed, jump, 5, pix, 1000, 8), orc.inject_ids(seed, jump, 6, pix, 1000, 8))
    assert not np.array_equal(orc.inject_ids(seed, 1, 5, pix, 1000, 8), orc.inject_ids(seed, 2, 5, pix, 1000, 8))


def test_injection_uniformity(orc):
    """Sanity: injected IDs over many pixels are uniform (chi-square, 15 dof)."""
    n = 16
    counts = np.zeros(n)
    for pix in range(4000):
        for i in orc.inject_ids(7, 1, 3, pix, n, 4):
            counts[i] += 1
    exp = counts.sum() / n
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 40.0


# ---------------------------------------------------------------- score pins
def _golden_eval(expr):
    if isinstance(expr, (int, float)):
        return float(expr)
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "exp": math.exp, "sqrt": math.sqrt}))


def _golden_sites(case):
    rows = [[_golden_eval(v) for v in s] for s in case["sites"]]
    return np.ascontiguousarray(np.array(rows, dtype=np.float64).T.astype(np.float32))


@pytest.mark.parametrize("case_idx", [0, 1, 2])
def test_golden_worked_scores(orc, case_idx):
    case = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["cases"][case_idx]
    S = _golden_sites(case)
    n = S.shape[1]
    for pix, sid, expr in case["scores"]:
        got = orc.score_pairs(S, n, case["W"], case["H"], [pix], [sid])[0]
        assert got == pytest.approx(_golden_eval(expr), abs=2e-7), (case["name"], pix, sid)


def test_golden_worked_blend(orc):
    case = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["cases"][0]
    S = _golden_sites(case)
    W, H = case["W"], case["H"]
    cand = np.full((H, W, 8), NONE, dtype=np.uint32)
    cand[:, :, 0] = 0
    cand[:, :, 1] = 1
    rgb = orc.render_fwd(S, 2, cand, W, H).reshape(-1, 3)
    exp = np.array([[_golden_eval(e) for e in row] for row in case["colours"]])
    # the fp64 oracle reads the float32-rounded log(2) and log(4)
    assert np.allclose(rgb, exp, atol=1e-7, rtol=0)


def test_score_matches_explicit_metric_matrix(orc):
    """d = s*sqrt(delta^T G delta) - s*r with G = e^a u u^T + e^-a v v^T built as a
    2x2 matrix (reading note, key design 1); det G = 1 (summary, section 4)."""
    W, H = 37, 23
    S = _sites(60, W, H, 11)
    S[synth.DX] *= 3.7  # |dir| != 1: the metric uses the normalised direction
    rng = np.random.default_rng(2)
    pix = rng.integers(0, W * H, 3000)
    ids = rng.integers(0, 60, 3000)
    got = orc.score_pairs(S, 60, W, H, pix, ids).astype(np.float64)
    S64 = S.astype(np.float64)
    dx, dy = S64[synth.DX, ids], S64[synth.DY, ids]
    nrm = np.hypot(dx, dy)
    u = np.stack([dx / nrm, dy / nrm], -1)
    v = np.stack([-u[:, 1], u[:, 0]], -1)
    a = S64[synth.A, ids]
    G = np.exp(a)[:, None, None] * u[:, :, None] * u[:, None, :] + np.exp(-a)[:, None, None] * v[:, :, None] * v[:, None, :]
    assert np.allclose(np.linalg.det(G), 1.0, atol=1e-12)
    cx, cy = (pix % W) + 0.5, (pix // W) + 0.5
    delta = np.stack([cx - S64[synth.X, ids], cy - S64[synth.Y, ids]], -1)
    q = np.sqrt(np.einsum("ni,nij,nj->n", delta, G, delta))
    s = 1.0 / max(W, H)
    exp = s * q - s * S64[synth.R, ids]
    assert np.allclose(got, exp, rtol=2e-6, atol=1e-6)


def test_score_isotropic_is_euclidean_and_symmetries(orc):
    W, H = 40, 30
    S = _sites(50, W, H, 12)
    S[synth.A] = 0.0
    rng = np.random.default_rng(3)
    pix = rng.integers(0, W * H, 2000)
    ids = rng.integers(0, 50, 2000)
    d0 = orc.score_pairs(S, 50, W, H, pix, ids).astype(np.float64)
    cx, cy = (pix % W) + 0.5, (pix // W) + 0.5
    euclid = np.hypot(cx - S[synth.X, ids], cy - S[synth.Y, ids]) / max(W, H) - S[synth.R, ids] / max(W, H)
    assert np.allclose(d0, euclid, rtol=1e-6, atol=1e-7)
    # u -> -u leaves d unchanged (bit-exact); (a, u) -> (-a, v) leaves it unchanged
    S2 = _sites(50, W, H, 13)
    d1 = orc.score_pairs(S2, 50, W, H, pix, ids)
    S3 = S2.copy()
    S3[synth.DX] *= -1
    S3[synth.DY] *= -1
    assert np.array_equal(orc.score_pairs(S3, 50, W, H, pix, ids), d1)
    S4 = S2.copy()
    S4[synth.DX], S4[synth.DY] = -S2[synth.DY], S2[synth.DX].copy()
    S4[synth.A] = -S2[synth.A]
    assert np.allclose(orc.score_pairs(S4, 50, W, H, pix, ids), d1, rtol=1e-6, atol=1e-7)
    # r shifts d by -s*r; s = 1/max(W,H)
    S5 = S2.copy()
    S5[synth.R] += 3.0
    assert np.allclose(orc.score_pairs(S5, 50, W, H, pix, ids), d1 - 3.0 / 40, atol=1e-6)
    # a degenerate direction is read as u = (1, 0)
    S6 = S2.copy()
    S6[synth.DX, :] = 0.0
    S6[synth.DY, :] = 0.0
    S7 = S2.copy()
    S7[synth.DX, :] = 1.0
    S7[synth.DY, :] = 0.0
    assert np.array_equal(orc.score_pairs(S6, 50, W, H, pix, ids), orc.score_pairs(S7, 50, W, H, pix, ids))


def test_score_unusable_entries_are_inf(orc):
    S = _sites(4, 8, 8, 1)
    S[synth.X, 2] = -1.0
    got = orc.score_pairs(S, 3, 8, 8, [0, 0, 0, 0], [NONE, 2, 3, 1])
    assert np.isinf(got[:3]).all() and np.isfinite(got[3])


# ------------------------------------------------------------ exact top-K pins
def test_exact_topk_is_euclidean_knn_when_isotropic(orc):
    """a = 0, r = 0: the score is the scaled Euclidean distance, so the exact top-K
    equals the 8 nearest neighbours from a k-d tree (scipy)."""
    from scipy.spatial import cKDTree

    W, H, n = 24, 20, 150
    S = _sites(n, W, H, 21)
    S[synth.A] = 0.0
    S[synth.R] = 0.0
    got = orc.topk_exact(S, n, W, H).reshape(-1, 8)
    cx, cy = _pix_centres(W, H)
    tree = cKDTree(np.stack([S[synth.X, :n], S[synth.Y, :n]], -1).astype(np.float64))
    dist, idx = tree.query(np.stack([cx, cy], -1), k=9)
    for p in range(W * H):
        if set(got[p]) != set(idx[p, :8]):
            assert dist[p, 8] - dist[p, 7] < 1e-4, p
        else:
            # stored in ascending score order
            assert list(got[p]) == list(idx[p, :8]) or np.ptp(dist[p, :8]) < 1e-4


def test_exact_topk_apollonius_order_and_inactive(orc):
    """a = 0: additively weighted (Apollonius) order |x - p| - r, inactive sites skipped,
    N < K pads with the sentinel."""
    W, H, n = 16, 12, 40
    S = _sites(n, W, H, 22)
    S[synth.A] = 0.0
    S[synth.X, ::3] = -1.0  # inactive
    got = orc.topk_exact(S, n, W, H).reshape(-1, 8)
    cx, cy = _pix_centres(W, H)
    act = np.where(S[synth.X, :n] >= 0)[0]
    for p in range(W * H):
        d = np.hypot(cx[p] - S[synth.X, act].astype(np.float64), cy[p] - S[synth.Y, act]) - S[synth.R, act]
        order = act[np.lexsort((act, d))][:8]
        assert list(got[p]) == list(order)
    # fewer active sites than K
    S2 = _sites(5, W, H, 23)
    got2 = orc.topk_exact(S2, 5, W, H).reshape(-1, 8)
    assert (got2[:, 5:] == NONE).all() and set(got2[0, :5]) == set(range(5))


def test_hard_render_is_argmin_colour(orc):
    W, H, n = 20, 20, 30
    S = _sites(n, W, H, 24)
    img = orc.hard_render(S, n, W, H).reshape(-1, 3)
    ex = orc.topk_exact(S, n, W, H).reshape(-1, 8)[:, 0]
    assert np.array_equal(img, S[synth.CR:synth.CB + 1, ex].T)


# ------------------------------------------------------------ propagation pins
def _worst_scores(orc, S, n, W, H, cand):
    """K-th (worst kept) score per pixel; +inf where the list is not full."""
    flat = cand.reshape(-1, 8)
    pix = np.repeat(np.arange(W * H), 8)
    sc = orc.score_pairs(S, n, W, H, pix, flat.ravel()).reshape(-1, 8)
    return sc.max(axis=1)


def test_propagate_exact_map_is_fixed_point(orc):
    W, H, n = 32, 24, 120
    S = _sites(n, W, H, 31)
    ex = orc.topk_exact(S, n, W, H)
    for jump in (1, 2, 8, 16):
        out = orc.propagate(S, n, ex, W, H, jump, 5, 99, 0)
        assert np.array_equal(out, ex)
    # with injection the exact map is still a fixed point (nothing can beat it)
    out = orc.propagate(S, n, ex, W, H, 1, 6, 99, 8)
    assert np.array_equal(out, ex)


def test_propagate_worst_score_never_increases_and_converges(orc):
    """Static sites: each pixel's K-th score is non-increasing over passes, and the
    coarse-to-fine schedule plus injection reaches the exact top-K (summary,
    section 4; press article section 3 reports >96% exact after 12-16 rounds)."""
    W, H, n = 48, 40, 200
    S = _sites(n, W, H, 32)
    cand = synth.empty_map(W, H)
    prev = np.full(W * H, np.inf)
    sched = orc.jump_schedule(W, H, 40)
    assert sched[:6] == [32, 16, 8, 4, 2, 1] and sched[-1] == 1
    ex = orc.topk_exact(S, n, W, H)
    exact_frac = []
    for t, k in enumerate(sched):
        cand = orc.propagate(S, n, cand, W, H, k, t, 4, 4)
        wst = _worst_scores(orc, S, n, W, H, cand)
        assert (wst <= prev).all()
        prev = wst
        exact_frac.append(np.mean([set(a) == set(b) for a, b in zip(cand.reshape(-1, 8), ex.reshape(-1, 8))]))
    assert exact_frac[15] > 0.9
    assert exact_frac[-1] > 0.995


def test_propagate_without_neighbours_sorts_own_list(orc):
    """jump beyond the image: only the own list and injection remain.  With no
    injection the result is the own list filtered, deduplicated and sorted by
    (score, ID) -- checked with numpy's lexsort."""
    W, H, n = 10, 7, 50
    S = _sites(n, W, H, 33)
    S[synth.X, 5] = -1.0
    cin = synth.random_map(W, H, n + 3, seed=5)  # includes IDs >= n, sentinels, dups
    out = orc.propagate(S, n, cin, W, H, 100, 0, 1, 0).reshape(-1, 8)
    for p in range(W * H):
        ids = np.array(sorted({int(i) for i in cin.reshape(-1, 8)[p] if i < n and S[synth.X, i] >= 0}), dtype=np.uint32)
        sc = orc.score_pairs(S, n, W, H, np.full(ids.size, p), ids)
        order = ids[np.lexsort((ids, sc))][:8]
        exp = np.full(8, NONE, dtype=np.uint32)
        exp[:order.size] = order
        assert np.array_equal(out[p], exp)


def test_propagate_neighbour_union_brute_force(orc):
    """Each pixel's output is the top-K of own + 4 neighbours at +-jump (skipped
    outside the image) + injected IDs: recomputed here by brute force."""
    W, H, n, m = 13, 9, 60, 4
    S = _sites(n, W, H, 34)
    cin = synth.random_map(W, H, n, seed=6)
    for jump in (1, 3, 8):
        out = orc.propagate(S, n, cin, W, H, jump, 77, 55, m).reshape(-1, 8)
        for p in range(W * H):
            r, c = divmod(p, W)
            cand = list(cin[r, c])
            for dc, dr in ((-jump, 0), (jump, 0), (0, -jump), (0, jump)):
                if 0 <= c + dc < W and 0 <= r + dr < H:
                    cand += list(cin[r + dr, c + dc])
            cand += list(orc.inject_ids(55, jump, 77, p, n, m))
            ids = np.array(sorted({int(i) for i in cand if i != NONE and i < n}), dtype=np.uint32)
            sc = orc.score_pairs(S, n, W, H, np.full(ids.size, p), ids)
            order = ids[np.lexsort((ids, sc))][:8]
            exp = np.full(8, NONE, dtype=np.uint32)
            exp[:order.size] = order
            assert np.array_equal(out[p], exp), (jump, p)
        u, cnt = orc.union_pixels(S, n, cin, W, H, jump, 77, 55, m, np.arange(W * H))
        for p in range(W * H):
            assert set(out[p][out[p] != NONE]) <= set(u[p, :cnt[p]])


def test_propagate_injection_only_from_empty(orc):
    W, H, n, m = 8, 8, 1000, 8
    S = _sites(n, W, H, 35)
    out = orc.propagate(S, n, synth.empty_map(W, H), W, H, 1, 3, 9, m).reshape(-1, 8)
    for p in range(W * H):
        inj = set(int(i) for i in orc.inject_ids(9, 1, 3, p, n, m))
        got = set(int(i) for i in out[p] if i != NONE)
        assert got == inj  # all 8 draws distinct here; an empty neighbourhood adds nothing else


# ---------------------------------------------------------------- forward pins
def _torch_forward(S64, n, cand, W, H):
    """A plain dense float64 PyTorch forward written from the pages' formulas with
    the explicit metric matrix (reading note, key designs 1-2)."""
    ids = torch.as_tensor(cand.reshape(-1, 8).astype(np.int64))
    valid = (ids != NONE) & (ids < n)
    idc = torch.where(valid, ids, torch.zeros_like(ids))
    px, py, lt, r = S64[0][idc], S64[1][idc], S64[2][idc], S64[3][idc]
    col = S64[4:7][:, idc].permute(1, 2, 0)
    dx, dy, a = S64[7][idc], S64[8][idc], S64[9][idc]
    valid = valid & (px >= 0)
    nrm = torch.sqrt(dx * dx + dy * dy)
    ux, uy = dx / nrm, dy / nrm
    vx, vy = -uy, ux
    E = torch.exp(a)
    g00 = E * ux * ux + vx * vx / E
    g01 = E * ux * uy + vx * vy / E
    g11 = E * uy * uy + vy * vy / E
    pix = torch.arange(W * H)
    cx = (pix % W).double()[:, None] + 0.5
    cy = (pix // W).double()[:, None] + 0.5
    ex, ey = cx - px, cy - py
    q = torch.sqrt(g00 * ex * ex + 2 * g01 * ex * ey + g11 * ey * ey)
    s = 1.0 / max(W, H)
    d = s * q - s * r
    logit = torch.where(valid, -torch.exp(lt) * d, torch.full_like(d, -math.inf))
    any_valid = valid.any(dim=1, keepdim=True)
    logit = torch.where(any_valid, logit, torch.zeros_like(logit))
    w = torch.softmax(logit, dim=1)
    w = torch.where(any_valid, w, torch.zeros_like(w))
    return (w[:, :, None] * col).sum(1)


def test_forward_matches_dense_torch(orc):
    W, H, n = 20, 16, 40
    S = _sites(n, W, H, 41)
    S[synth.DX] *= 2.5
    S[synth.X, 3] = -1.0
    cand = synth.random_map(W, H, n + 2, seed=7)
    cand[0, 0, :] = NONE
    got = orc.render_fwd(S, n, cand, W, H).reshape(-1, 3)
    ref = _torch_forward(torch.as_tensor(S.astype(np.float64)), n, cand, W, H).numpy()
    assert np.allclose(got, ref, atol=1e-12, rtol=1e-10)
    assert np.array_equal(got[0], [0, 0, 0])  # empty list renders 0


def test_forward_limits(orc):
    W, H, n = 16, 16, 64
    S = _sites(n, W, H, 42)
    ex = orc.topk_exact(S, n, W, H)
    # weights sum to one: with every colour = 1 the render is exactly 1
    S1 = S.copy()
    S1[synth.CR:synth.CB + 1] = 1.0
    assert np.allclose(orc.render_fwd(S1, n, ex, W, H), 1.0, atol=1e-14)
    # tau -> 0: the plain mean of the list's colours
    S2 = S.copy()
    S2[synth.LOGTAU] = -40.0
    mean = S[synth.CR:synth.CB + 1][:, ex.reshape(-1, 8)].mean(axis=2).T
    assert np.allclose(orc.render_fwd(S2, n, ex, W, H).reshape(-1, 3), mean, atol=1e-9)
    # equal large tau: the hard (argmin) render, i.e. the Apollonius diagram
    S3 = S.copy()
    S3[synth.LOGTAU] = 14.0
    hard = orc.hard_render(S, n, W, H)
    soft = orc.render_fwd(S3, n, ex, W, H)
    close = np.abs(soft - hard).max(axis=2) < 1e-6
    assert close.mean() > 0.97
    # a single valid entry renders its colour exactly
    one = synth.empty_map(W, H)
    one[:, :, 3] = 5
    assert np.allclose(orc.render_fwd(S, n, one, W, H).reshape(-1, 3), S[synth.CR:synth.CB + 1, 5][None, :], atol=0)


# --------------------------------------------------------------- backward pins
def test_backward_matches_torch_autograd(orc):
    W, H, n = 18, 14, 36
    S = _sites(n, W, H, 51)
    S[synth.DX] *= 1.7
    S[synth.X, 4] = -1.0
    cand = synth.random_map(W, H, n + 2, seed=8)
    tgt = synth.pixel_noise(W, H, 9, 0.3) + 0.5
    g, loss = orc.render_bwd(S, n, cand, tgt, W, H)
    St = torch.tensor(S.astype(np.float64), requires_grad=True)
    c = _torch_forward(St, n, cand, W, H)
    L = ((c - torch.as_tensor(tgt.reshape(-1, 3).astype(np.float64))) ** 2).sum()
    L.backward()
    assert loss == pytest.approx(L.item(), rel=1e-12)
    ref = St.grad.numpy()
    for j in range(10):
        assert np.allclose(g[j], ref[j], rtol=1e-8, atol=1e-10), j


def test_backward_matches_central_differences(orc):
    W, H, n = 12, 10, 20
    S = _sites(n, W, H, 52).astype(np.float64)
    cand = orc.topk_exact(S.astype(np.float32), n, W, H)
    tgt = synth.pixel_noise(W, H, 10, 0.3) + 0.5
    g, _ = orc.render_bwd(S, n, cand, tgt, W, H)

    def loss(S_):
        c = orc.render_fwd(S_, n, cand, W, H)
        return ((c - tgt.astype(np.float64)) ** 2).sum()

    rng = np.random.default_rng(4)
    for j in range(10):
        for i in rng.choice(n, 4, replace=False):
            h = 1e-6 * max(1.0, abs(S[j, i]))
            Sp, Sm = S.copy(), S.copy()
            Sp[j, i] += h
            Sm[j, i] -= h
            fd = (loss(Sp) - loss(Sm)) / (2 * h)
            assert fd == pytest.approx(g[j, i], rel=1e-5, abs=1e-7), (j, i)


def _distinct_map(W, H, n, seed, p_invalid=0.2):
    """Lists of 8 distinct IDs (as propagation produces), some entries sentinel."""
    rng = np.random.default_rng(seed)
    m = np.stack([rng.permutation(n)[:8] for _ in range(W * H)]).astype(np.uint32)
    m[rng.random(m.shape) < p_invalid] = NONE
    return m.reshape(H, W, 8)


def test_backward_colour_sum_and_removal_delta(orc):
    W, H, n = 16, 12, 30
    S = _sites(n, W, H, 53).astype(np.float64)
    cand = _distinct_map(W, H, n, 11)
    cand[2, 3, :] = NONE
    cand[4, 4, 1:] = NONE  # a sole contributor: removing it leaves an empty list
    tgt = synth.pixel_noise(W, H, 12, 0.3) + 0.5
    g, loss = orc.render_bwd(S, n, cand, tgt, W, H)
    c = orc.render_fwd(S, n, cand, W, H)
    err = ((c - tgt) ** 2).sum(axis=2)
    assert loss == pytest.approx(err.sum(), rel=1e-12)
    nonempty = (cand != NONE).any(axis=2)
    # sum over sites of dL/dc equals sum over (non-empty) pixels of 2 (c - t)
    for ch in range(3):
        assert g[4 + ch].sum() == pytest.approx((2 * (c - tgt))[..., ch][nonempty].sum(), rel=1e-10, abs=1e-10)
    # removal delta: drop each entry, re-render the pixel, difference of squared errors
    rd = np.zeros(n)
    for k in range(8):
        mk = cand.copy()
        mk[:, :, k] = NONE
        ck = orc.render_fwd(S, n, mk, W, H)
        dk = (((ck - tgt) ** 2).sum(axis=2) - err).ravel()
        ids = cand.reshape(-1, 8)[:, k]
        ok = ids != NONE
        np.add.at(rd, ids[ok].astype(np.int64), dk[ok])
    assert np.allclose(g[10, :n], rd, rtol=1e-9, atol=1e-12)


def test_backward_accumulates_and_skips_inactive(orc):
    W, H, n = 8, 8, 12
    S = _sites(n, W, H, 54).astype(np.float64)
    S[0, 2] = -1.0
    cand = orc.topk_exact(S.astype(np.float32), n, W, H)
    cand[0, 0, 0] = 2  # an inactive site in a list is skipped
    tgt = synth.pixel_noise(W, H, 13, 0.3) + 0.5
    g1, l1 = orc.render_bwd(S, n, cand, tgt, W, H)
    assert (g1[:, 2] == 0).all()
    g2, l2 = orc.render_bwd(S, n, cand, tgt, W, H, grad=g1.copy())
    assert np.allclose(g2, 2 * g1) and l2 == pytest.approx(l1)


# ------------------------------------------------------------------- Adam pins
LR = np.array([0.1, 0.1, 0.02, 0.05, 0.01, 0.01, 0.01, 0.02, 0.02, 0.02])


def test_adam_first_step_closed_form(orc):
    W, H, n = 50, 40, 16
    S = _sites(n, W, H, 61).astype(np.float64)
    S[0, 3] = -1.0
    rng = np.random.default_rng(5)
    G = np.zeros((11, n))
    G[:10] = rng.normal(0, 1, (10, n)) * 100
    G[10] = 7.0
    P = W * H
    p, m, v, g = S.copy(), np.zeros((10, n)), np.zeros((10, n)), G.copy()
    orc.adam_step(p, m, v, g, n, 1, P, LR, 0.9, 0.999, 1e-8, W, H)
    gh = G[:10] / P
    exp = S - LR[:, None] * gh / (np.abs(gh) + 1e-8)
    exp[0] = np.clip(exp[0], 0, W)
    exp[1] = np.clip(exp[1], 0, H)
    act = np.arange(n) != 3
    assert np.allclose(p[:, act], exp[:, act], rtol=1e-12, atol=1e-12)
    assert np.array_equal(p[:, 3], S[:, 3]) and (m[:, 3] == 0).all()
    assert (g[:10] == 0).all() and (g[10] == 7.0).all()


def test_adam_matches_torch_optim(orc):
    W, H, n = 64, 64, 32
    S = _sites(n, W, H, 62).astype(np.float64)
    S[0] = np.clip(S[0], 20, 44)
    S[1] = np.clip(S[1], 20, 44)
    P = W * H
    rng = np.random.default_rng(6)
    params = [torch.tensor(S[j].copy(), requires_grad=True) for j in range(10)]
    opt = torch.optim.Adam([{"params": [params[j]], "lr": float(LR[j])} for j in range(10)],
                           betas=(0.9, 0.999), eps=1e-8)
    p, m, v = S.copy(), np.zeros((10, n)), np.zeros((10, n))
    for t in range(1, 6):
        G = np.zeros((11, n))
        G[:10] = rng.normal(0, 50, (10, n))
        for j in range(10):
            params[j].grad = torch.tensor(G[j] / P)
        opt.step()
        orc.adam_step(p, m, v, G, n, t, P, LR, 0.9, 0.999, 1e-8, W, H)
        ref = np.stack([q.detach().numpy() for q in params])
        assert np.allclose(p, ref, rtol=1e-12, atol=1e-12), t


def test_adam_clamps_position_and_zeroes_nonfinite(orc):
    W, H, n = 10, 10, 4
    S = _sites(n, W, H, 63).astype(np.float64)
    S[0, 0] = 0.01
    S[1, 1] = 9.99
    G = np.zeros((11, n))
    G[0, 0] = 1e3   # pushes x of site 0 below 0
    G[1, 1] = -1e3  # pushes y of site 1 above H
    G[2, 2] = np.nan
    p, m, v = S.copy(), np.zeros((10, n)), np.zeros((10, n))
    orc.adam_step(p, m, v, G, n, 1, W * H, LR, 0.9, 0.999, 1e-8, W, H)
    assert p[0, 0] == 0.0 and p[1, 1] == float(H)
    assert p[2, 2] == S[2, 2] and m[2, 2] == 0 and np.isfinite(p).all()
