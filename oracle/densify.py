"""Oracle of the host-side budget control (densify / prune).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Written from the pages:
paperlayer.ai summary, Appendix B.5 (a site's error energy over a power of its
mass ranks it for splitting; a split places two children on either side of the
parent along an axis from the error-weighted covariance, or from the luminance
gradient when that is unusable; the children read their colour from the target,
shrink r and log tau and start with zero Adam moments; the sites whose removal
costs least are dropped by moving them to (-1, -1)), the reading note's key
design 4 and the press article's section 4.  The pages give no constants; the
rules and defaults below are our reading, each stated at the point where it is
applied.

PARITY UNPINNED against the pages: there is no second source for these rules;
the tests pin only invariants (counts, symmetry of the children about the
parent, fresh Adam state, pruned positions, seeding) and hand-built cases.
"""
from __future__ import annotations

import math

import numpy as np

X, Y, LOGTAU, R, CR, CG, CB = 0, 1, 2, 3, 4, 5, 6
NONE = 0xFFFFFFFF


def _luma(t, c, r):
    H, W, _ = t.shape
    c = min(max(c, 0), W - 1)
    r = min(max(r, 0), H - 1)
    q = t[r, c].astype(np.float64)
    return 0.299 * q[0] + 0.587 * q[1] + 0.114 * q[2]


def _pix(x, n):
    return min(max(int(math.floor(x)), 0), n - 1)


def densify_prune(sites, m, v, n_slots, capacity, stats, removal, cand, W, H, target, split_frac=0.05,
                  prune_frac=0.05, alpha=0.5, min_mass=1.0, shrink=0.85, cell=1):
    """In place on float32 sites/m/v [10][stride] and uint32 cand [Hm][Wm][8]
    (cells of `cell` x `cell` pixels, Wm = ceil(W / cell); per pixel when 1).

    Returns (n_slots, n_split, n_pruned, short_of_slots)."""
    Wm, Hm = -(-W // cell), -(-H // cell)
    assert cand.shape == (Hm, Wm, 8)
    stride = sites.shape[1]
    active = [i for i in range(n_slots) if not (sites[X, i] < 0)]
    A = len(active)
    n_split = int(math.floor(split_frac * A))
    n_prune = int(math.floor(prune_frac * A))
    # split set: score = energy / max(mass, min_mass)^alpha, largest first, ties -> lower ID
    scored = []
    for i in active:
        mass, energy = float(stats[i, 0]), float(stats[i, 1])
        S = energy / max(mass, min_mass) ** alpha
        if math.isfinite(S) and S > 0:
            scored.append((-S, i))
    scored.sort()
    split = [i for _, i in scored[:n_split]]
    in_split = set(split)
    # prune set: smallest removal delta among the rest, ties -> lower ID
    cands = sorted((float(removal[i]), i) for i in active if i not in in_split and math.isfinite(removal[i]))
    pruned = 0
    for _, i in cands[:n_prune]:
        sites[X, i] = -1.0
        sites[Y, i] = -1.0
        m[:, i] = 0.0
        v[:, i] = 0.0
        pruned += 1
    free = [i for i in range(n_slots) if sites[X, i] < 0]
    count = n_slots
    done = 0
    short = False
    for i in split:
        if free:
            b = free.pop(0)
        elif count < capacity:
            b = count
            count += 1
        else:
            short = True
            break
        mass, E = float(stats[i, 0]), float(stats[i, 1])
        axis = None
        if mass >= min_mass and E > 0:
            mx, my = stats[i, 2] / E, stats[i, 3] / E
            C = np.array([[stats[i, 4] / E - mx * mx, stats[i, 5] / E - mx * my],
                          [stats[i, 5] / E - mx * my, stats[i, 6] / E - my * my]], dtype=np.float64)
            lam, vec = np.linalg.eigh(C)
            if math.isfinite(lam[1]) and lam[1] > 0:
                e = vec[:, 1]
                if lam[0] == lam[1]:  # isotropic: the axis is a free choice, take +x
                    e = np.array([1.0, 0.0])
                elif e[0] < 0 or (e[0] == 0 and e[1] < 0):  # orientation: x > 0, else +y
                    e = -e
                axis = 0.5 * math.sqrt(lam[1]) * e
        if axis is None:
            c, r = _pix(float(sites[X, i]), W), _pix(float(sites[Y, i]), H)
            gx = (_luma(target, c + 1, r - 1) + 2 * _luma(target, c + 1, r) + _luma(target, c + 1, r + 1)) - \
                 (_luma(target, c - 1, r - 1) + 2 * _luma(target, c - 1, r) + _luma(target, c - 1, r + 1))
            gy = (_luma(target, c - 1, r + 1) + 2 * _luma(target, c, r + 1) + _luma(target, c + 1, r + 1)) - \
                 (_luma(target, c - 1, r - 1) + 2 * _luma(target, c, r - 1) + _luma(target, c + 1, r - 1))
            gn = math.hypot(gx, gy)
            g = np.array([gx / gn, gy / gn]) if gn > 0 else np.array([1.0, 0.0])
            axis = 0.5 * math.sqrt(max(mass, 1.0) / math.pi) * g
        parent = sites[:, i].astype(np.float64).copy()
        for slot, sign in ((i, -1.0), (b, 1.0)):
            sites[:, slot] = parent.astype(np.float32)
            m[:, slot] = 0.0
            v[:, slot] = 0.0
            x = min(max(parent[X] + sign * axis[0], 0.0), float(W))
            y = min(max(parent[Y] + sign * axis[1], 0.0), float(H))
            sites[X, slot] = x
            sites[Y, slot] = y
            sites[R, slot] = np.float32(parent[R]) * np.float32(shrink)
            sites[LOGTAU, slot] = np.float32(parent[LOGTAU]) + np.float32(math.log(np.float32(shrink)))
            sites[CR:CB + 1, slot] = target[_pix(y, H), _pix(x, W)]
        # child B enters the list of its pixel's map entry and of the 4 neighbour
        # entries, in the last place -- except a list that already names b (a slot
        # freed by this call's pruning keeps its ID in lists near its old place):
        # a candidate list names distinct sites
        bc, br = _pix(float(sites[X, b]), W) // cell, _pix(float(sites[Y, b]), H) // cell
        for dc, dr in ((0, 0), (-1, 0), (1, 0), (0, -1), (0, 1)):
            c, r = bc + dc, br + dr
            if 0 <= c < Wm and 0 <= r < Hm and not np.any(cand[r, c] == b):
                cand[r, c, 7] = b
        done += 1
    return count, done, pruned, short
