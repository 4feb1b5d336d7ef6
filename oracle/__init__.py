"""ctypes binding of the plain CPU oracle (``sad_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the CPU-baseline leg of ``bench.py``; never by the product path.  It
imports nothing from the product package.

Every function mirrors one routine of ``sad_oracle.c``; see that file for the
definitions and the passages of the pages each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sad_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

K = 8
NONE = 0xFFFFFFFF
NPARAM = 10
NACC = 11

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, OpenMP, no FP contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int)
        c_int, c_u32, c_long, c_dbl = ctypes.c_int, ctypes.c_uint32, ctypes.c_long, ctypes.c_double
        sig = {
            "orc_version": (c_int, []),
            "orc_set_threads": (None, [c_int]),
            "orc_get_threads": (c_int, []),
            "orc_pcg_hash": (c_u32, [c_u32]),
            "orc_xorshift32": (c_u32, [c_u32]),
            "orc_pass_word": (c_u32, [c_int, c_u32]),
            "orc_inject_ids": (None, [c_u32, c_int, c_u32, c_u32, c_u32, c_int, u32p]),
            "orc_score_pairs": (None, [f32p, c_int, c_int, c_int, c_int, c_int, u32p, u32p, c_long, f32p]),
            "orc_topk_exact": (None, [f32p, c_int, c_int, c_int, c_int, c_int, u32p]),
            "orc_topk_exact_pixels": (None, [f32p, c_int, c_int, c_int, c_int, c_int, u32p, c_long, u32p]),
            "orc_hard_render": (None, [f32p, c_int, c_int, c_int, c_int, f32p]),
            "orc_propagate": (None, [f32p, c_int, c_int, u32p, u32p, c_int, c_int, c_int, c_int, c_u32, c_u32,
                                     c_int]),
            "orc_propagate_pixels": (None, [f32p, c_int, c_int, u32p, c_int, c_int, c_int, c_int, c_u32, c_u32,
                                            c_int, u32p, c_long, u32p]),
            "orc_union_pixels": (None, [f32p, c_int, u32p, c_int, c_int, c_int, c_int, c_u32, c_u32, c_int, u32p,
                                        c_long, u32p, i32p]),
            "orc_max_union": (c_int, []),
            "orc_render_fwd": (None, [f64p, c_int, c_int, u32p, c_int, c_int, c_int, f64p]),
            "orc_render_fwd_pixels": (None, [f64p, c_int, c_int, u32p, c_int, c_int, c_int, u32p, c_long, f64p]),
            "orc_render_bwd": (None, [f64p, c_int, c_int, u32p, f32p, c_int, c_int, c_int, f64p, f64p]),
            "orc_adam_step": (None, [f64p, f64p, f64p, f64p, c_int, c_int, c_int, c_int, f64p, c_dbl, c_dbl,
                                     c_dbl, c_int, c_int]),
            "orc_densify_stats": (None, [f64p, c_int, c_int, u32p, f32p, c_int, c_int, c_int, f64p]),
            "orc_query_points": (None, [f64p, c_int, c_int, u32p, c_int, c_int, c_int, f32p, c_long, f64p]),
            "orc_jfa_seed": (None, [f32p, c_int, c_int, c_int, c_int, c_int, u32p]),
            "orc_jfa_pass": (None, [f32p, c_int, c_int, u32p, u32p, c_int, c_int, c_int, c_int]),
            "orc_jfa_pass_pixels": (None, [f32p, c_int, c_int, u32p, c_int, c_int, c_int, c_int, u32p, c_long,
                                           u32p]),
            "orc_jfa_union_pixels": (None, [f32p, c_int, u32p, c_int, c_int, c_int, c_int, u32p, c_long, u32p,
                                            i32p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _u32(a):
    return np.ascontiguousarray(a, dtype=np.uint32)


def map_shape(W: int, H: int, cell: int = 1) -> tuple:
    """Shape of a candidate map on the grid of `cell` x `cell` pixel cells."""
    return (-(-H // cell), -(-W // cell), K)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return lib().orc_get_threads()


# ------------------------------------------------------------------ RNG
def pcg_hash(v: int) -> int:
    return lib().orc_pcg_hash(v & 0xFFFFFFFF)


def xorshift32(x: int) -> int:
    return lib().orc_xorshift32(x & 0xFFFFFFFF)


def pass_word(jump: int, pass_index: int) -> int:
    return lib().orc_pass_word(jump, pass_index & 0xFFFFFFFF)


def inject_ids(seed: int, jump: int, pass_index: int, pix: int, n_slots: int, m: int) -> np.ndarray:
    out = np.empty(max(m, 1), dtype=np.uint32)
    lib().orc_inject_ids(seed & 0xFFFFFFFF, jump, pass_index & 0xFFFFFFFF, pix, n_slots, m, _p(out, ctypes.c_uint32))
    return out[:m]


# ---------------------------------------------------------------- score
def score_pairs(sites, n_slots, W, H, pix, ids, cell=1) -> np.ndarray:
    """Selection scores of (map entry, ID) pairs (cell centres for cell > 1)."""
    S = _f32(sites)
    pix = _u32(pix).ravel()
    ids = _u32(ids).ravel()
    out = np.empty(pix.size, dtype=np.float32)
    lib().orc_score_pairs(_p(S, ctypes.c_float), n_slots, S.shape[1], W, H, cell, _p(pix, ctypes.c_uint32),
                          _p(ids, ctypes.c_uint32), pix.size, _p(out, ctypes.c_float))
    return out


# ------------------------------------------------------------ exact top-K
def topk_exact(sites, n_slots, W, H, cell=1) -> np.ndarray:
    S = _f32(sites)
    out = np.empty(map_shape(W, H, cell), dtype=np.uint32)
    lib().orc_topk_exact(_p(S, ctypes.c_float), n_slots, S.shape[1], W, H, cell, _p(out, ctypes.c_uint32))
    return out


def topk_exact_pixels(sites, n_slots, W, H, pix, cell=1) -> np.ndarray:
    S = _f32(sites)
    pix = _u32(pix).ravel()
    out = np.empty((pix.size, K), dtype=np.uint32)
    lib().orc_topk_exact_pixels(_p(S, ctypes.c_float), n_slots, S.shape[1], W, H, cell, _p(pix, ctypes.c_uint32),
                                pix.size, _p(out, ctypes.c_uint32))
    return out


def hard_render(sites, n_slots, W, H) -> np.ndarray:
    S = _f32(sites)
    out = np.empty((H, W, 3), dtype=np.float32)
    lib().orc_hard_render(_p(S, ctypes.c_float), n_slots, S.shape[1], W, H, _p(out, ctypes.c_float))
    return out


# ------------------------------------------------------------ propagation
def propagate(sites, n_slots, cin, W, H, jump, pass_index, seed, m, cell=1) -> np.ndarray:
    S = _f32(sites)
    cin = _u32(cin)
    assert cin.shape == map_shape(W, H, cell)
    out = np.empty_like(cin)
    lib().orc_propagate(_p(S, ctypes.c_float), n_slots, S.shape[1], _p(cin, ctypes.c_uint32),
                        _p(out, ctypes.c_uint32), W, H, cell, jump, pass_index & 0xFFFFFFFF, seed & 0xFFFFFFFF, m)
    return out


def propagate_pixels(sites, n_slots, cin, W, H, jump, pass_index, seed, m, pix, cell=1) -> np.ndarray:
    S = _f32(sites)
    cin = _u32(cin)
    assert cin.shape == map_shape(W, H, cell)
    pix = _u32(pix).ravel()
    out = np.empty((pix.size, K), dtype=np.uint32)
    lib().orc_propagate_pixels(_p(S, ctypes.c_float), n_slots, S.shape[1], _p(cin, ctypes.c_uint32), W, H, cell,
                               jump, pass_index & 0xFFFFFFFF, seed & 0xFFFFFFFF, m, _p(pix, ctypes.c_uint32),
                               pix.size, _p(out, ctypes.c_uint32))
    return out


def union_pixels(sites, n_slots, cin, W, H, jump, pass_index, seed, m, pix, cell=1):
    S = _f32(sites)
    cin = _u32(cin)
    assert cin.shape == map_shape(W, H, cell)
    pix = _u32(pix).ravel()
    mu = lib().orc_max_union()
    out = np.empty((pix.size, mu), dtype=np.uint32)
    cnt = np.empty(pix.size, dtype=np.int32)
    lib().orc_union_pixels(_p(S, ctypes.c_float), n_slots, _p(cin, ctypes.c_uint32), W, H, cell, jump,
                           pass_index & 0xFFFFFFFF, seed & 0xFFFFFFFF, m, _p(pix, ctypes.c_uint32), pix.size,
                           _p(out, ctypes.c_uint32), _p(cnt, ctypes.c_int))
    return out, cnt


def jump_schedule(W: int, H: int, n_iters: int, cell: int = 1) -> list:
    """Jumps B/2, B/4, ..., 1, then 1; B = 2^ceil(log2 max(Wm, Hm)) over the map's
    entries (Wm = ceil(W / cell), Hm likewise).

    (pages: paperlayer.ai summary, section 4 "Candidate maintenance"; B is our
    reading, since the pages do not define it.)
    """
    W, H = -(-W // cell), -(-H // cell)
    B = 1 << max(0, (max(W, H) - 1).bit_length())
    out, k = [], B // 2
    for _ in range(n_iters):
        out.append(max(k, 1))
        k //= 2
    return out


# ---------------------------------------------------------------- render
def render_fwd(sites, n_slots, cand, W, H, cell=1) -> np.ndarray:
    S = _f64(sites)
    cand = _u32(cand)
    assert cand.shape == map_shape(W, H, cell)
    out = np.empty((H, W, 3), dtype=np.float64)
    lib().orc_render_fwd(_p(S, ctypes.c_double), n_slots, S.shape[1], _p(cand, ctypes.c_uint32), W, H, cell,
                         _p(out, ctypes.c_double))
    return out


def render_fwd_pixels(sites, n_slots, cand, W, H, pix, cell=1) -> np.ndarray:
    S = _f64(sites)
    cand = _u32(cand)
    assert cand.shape == map_shape(W, H, cell)
    pix = _u32(pix).ravel()
    out = np.empty((pix.size, 3), dtype=np.float64)
    lib().orc_render_fwd_pixels(_p(S, ctypes.c_double), n_slots, S.shape[1], _p(cand, ctypes.c_uint32), W, H, cell,
                                _p(pix, ctypes.c_uint32), pix.size, _p(out, ctypes.c_double))
    return out


def render_bwd(sites, n_slots, cand, target, W, H, grad=None, cell=1):
    """Returns (grad float64 [11][stride], loss_sum).  Accumulates into `grad` if given."""
    S = _f64(sites)
    cand = _u32(cand)
    assert cand.shape == map_shape(W, H, cell)
    T = _f32(target)
    if grad is None:
        grad = np.zeros((NACC, S.shape[1]), dtype=np.float64)
    assert grad.dtype == np.float64 and grad.flags["C_CONTIGUOUS"] and grad.shape == (NACC, S.shape[1])
    loss = np.zeros(1, dtype=np.float64)
    lib().orc_render_bwd(_p(S, ctypes.c_double), n_slots, S.shape[1], _p(cand, ctypes.c_uint32),
                         _p(T, ctypes.c_float), W, H, cell, _p(grad, ctypes.c_double), _p(loss, ctypes.c_double))
    return grad, float(loss[0])


# ------------------------------------------------------------------ Adam
def adam_step(params, m, v, grad, n_slots, step, n_pixels, lr, b1, b2, eps, W, H) -> None:
    """In place on float64 arrays params/m/v [10][stride] and grad [11][stride]."""
    for a in (params, m, v, grad):
        assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    lr = _f64(lr)
    lib().orc_adam_step(_p(params, ctypes.c_double), _p(m, ctypes.c_double), _p(v, ctypes.c_double),
                        _p(grad, ctypes.c_double), n_slots, params.shape[1], step, n_pixels,
                        _p(lr, ctypes.c_double), b1, b2, eps, W, H)


# ------------------------------------------------------------ budget control
def densify_stats(sites, n_slots, cand, target, W, H, stats=None, cell=1):
    """Per-site mass, energy and error-weighted moments, float64 [stride][8] (+=)."""
    S = _f64(sites)
    cand = _u32(cand)
    assert cand.shape == map_shape(W, H, cell)
    T = _f32(target)
    if stats is None:
        stats = np.zeros((S.shape[1], 8), dtype=np.float64)
    assert stats.dtype == np.float64 and stats.flags["C_CONTIGUOUS"] and stats.shape == (S.shape[1], 8)
    lib().orc_densify_stats(_p(S, ctypes.c_double), n_slots, S.shape[1], _p(cand, ctypes.c_uint32),
                            _p(T, ctypes.c_float), W, H, cell, _p(stats, ctypes.c_double))
    return stats


def query_points(sites, n_slots, cand, W, H, pts, cell=1) -> np.ndarray:
    """Blend at arbitrary points (float32 [n][2], px) with the list of each point's
    map entry; float64 [n][3]."""
    S = _f64(sites)
    cand = _u32(cand)
    assert cand.shape == map_shape(W, H, cell)
    P = _f32(pts).reshape(-1, 2)
    out = np.empty((P.shape[0], 3), dtype=np.float64)
    lib().orc_query_points(_p(S, ctypes.c_double), n_slots, S.shape[1], _p(cand, ctypes.c_uint32), W, H, cell,
                           _p(P, ctypes.c_float), P.shape[0], _p(out, ctypes.c_double))
    return out


# ------------------------------------------------------------ JFA prepass
def jfa_seed(sites, n_slots, W, H, cell=1) -> np.ndarray:
    """Seed pass: each active site into the list of its map entry, <= 4 per entry."""
    S = _f32(sites)
    out = np.empty(map_shape(W, H, cell), dtype=np.uint32)
    lib().orc_jfa_seed(_p(S, ctypes.c_float), n_slots, S.shape[1], W, H, cell, _p(out, ctypes.c_uint32))
    return out


def jfa_pass(sites, n_slots, cin, W, H, step, cell=1) -> np.ndarray:
    S = _f32(sites)
    cin = _u32(cin)
    assert cin.shape == map_shape(W, H, cell)
    out = np.empty_like(cin)
    lib().orc_jfa_pass(_p(S, ctypes.c_float), n_slots, S.shape[1], _p(cin, ctypes.c_uint32),
                       _p(out, ctypes.c_uint32), W, H, cell, step)
    return out


def jfa_pass_pixels(sites, n_slots, cin, W, H, step, pix, cell=1) -> np.ndarray:
    S = _f32(sites)
    cin = _u32(cin)
    assert cin.shape == map_shape(W, H, cell)
    pix = _u32(pix).ravel()
    out = np.empty((pix.size, K), dtype=np.uint32)
    lib().orc_jfa_pass_pixels(_p(S, ctypes.c_float), n_slots, S.shape[1], _p(cin, ctypes.c_uint32), W, H, cell,
                              step, _p(pix, ctypes.c_uint32), pix.size, _p(out, ctypes.c_uint32))
    return out


def jfa_union_pixels(sites, n_slots, cin, W, H, step, pix, cell=1):
    S = _f32(sites)
    cin = _u32(cin)
    assert cin.shape == map_shape(W, H, cell)
    pix = _u32(pix).ravel()
    mu = lib().orc_max_union()
    out = np.empty((pix.size, mu), dtype=np.uint32)
    cnt = np.empty(pix.size, dtype=np.int32)
    lib().orc_jfa_union_pixels(_p(S, ctypes.c_float), n_slots, _p(cin, ctypes.c_uint32), W, H, cell, step,
                               _p(pix, ctypes.c_uint32), pix.size, _p(out, ctypes.c_uint32),
                               _p(cnt, ctypes.c_int))
    return out, cnt


def jfa_steps(W: int, H: int, cell: int = 1) -> list:
    """The prepass's steps: B/2, ..., 1 with B = 2^ceil(log2 max(Wm, Hm)) over the map's
    entries (ceil(log2) passes)."""
    W, H = -(-W // cell), -(-H // cell)
    B = 1 << max(0, (max(W, H) - 1).bit_length())
    out, k = [], B // 2
    while k >= 1:
        out.append(k)
        k //= 2
    return out


from .densify import densify_prune  # noqa: E402  (pure Python, no C)
from .packed import pack_words, rounded_sites  # noqa: E402  (numpy only)
from .evalpack import eval_decode, eval_encode  # noqa: E402  (numpy only)
