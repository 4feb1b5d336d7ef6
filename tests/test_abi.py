"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/sad.h declares, and rejects bad arguments before launching
anything (the dummy pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import soft_voronoi_render_amd as sad

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sad.h")

ERR_ARG, ERR_ALIGN = -1, -2


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sad.LIB_PATH):
        sad.build()
    return sad.lib()


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sad_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_hot_path():
    names = _declared()
    for fn in ("sad_topk_propagate", "sad_render_fwd", "sad_render_bwd", "sad_adam_step", "sad_densify_prune",
               "sad_topk_propagate_rec", "sad_render_fwd_rec", "sad_render_bwd_rec", "sad_adam_step_rec",
               "sad_densify_prune_stats", "sad_apply_seeds", "sad_topk_exact", "sad_topk_exact_at",
               "sad_site_records", "sad_abi_version", "sad_status_string"):
        assert fn in names


def test_header_signatures_of_the_site_buffer_calls():
    """The five calls of the iteration on the site buffer take the argument lists
    of the boundary: site planes with their stride, gradient planes, a scalar loss."""
    txt = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    sig = lambda fn: re.sub(r"\s+", " ", re.search(r"int " + fn + r"\((.*?)\);", txt, flags=re.S).group(1))
    assert sig("sad_topk_propagate") == ("const float *sites, int n_slots, int stride, const uint32_t *cand_in, "
                                         "uint32_t *cand_out, int W, int H, int jump, uint32_t pass_index, "
                                         "uint32_t seed, int n_inject, void *stream")
    assert sig("sad_render_fwd") == ("const float *sites, int n_slots, int stride, const uint32_t *cand, int W, "
                                     "int H, float *out_rgb, void *stream")
    assert sig("sad_render_bwd") == ("const float *sites, int n_slots, int stride, const uint32_t *cand, "
                                     "const float *target, int W, int H, float *grad, float *loss_sum, "
                                     "void *stream")
    assert sig("sad_adam_step") == ("float *sites, float *m, float *v, float *grad, int n_slots, int stride, "
                                    "int step, int n_pixels, const sad_adam_cfg *cfg, void *stream")
    assert sig("sad_densify_prune") == ("float *sites, float *m, float *v, float *removal, int *n_slots, "
                                        "int capacity, int stride, uint32_t *cand, int W, int H, "
                                        "const float *target, const sad_budget_cfg *cfg, uint64_t seed")


def test_library_exports_every_declared_symbol(L):
    for fn in _declared():
        assert hasattr(L, fn), fn
    assert set(_declared()) == set(sad.EXPORTED)


def test_abi_version_and_status_strings(L):
    assert L.sad_abi_version() == 7
    assert L.sad_status_string(0) == b"ok"
    assert L.sad_status_string(ERR_ALIGN) == b"misaligned pointer"
    assert L.sad_status_string(12345) == b"unknown status"


P = 0x10000  # a 16-byte aligned dummy address; never dereferenced on these paths
Q = 0x90000


def test_propagate_rejects_bad_arguments(L):
    f = L.sad_topk_propagate_rec
    ok = dict(rec=P, fmt=0, scr=None, n=4, a=P, b=Q, W=16, H=16, cell=1, jump=1, pidx=0, seed=0, m=4)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["rec"], a["fmt"], a["scr"], a["n"], a["a"], a["b"], a["W"], a["H"], a["cell"], a["jump"], a["pidx"],
                 a["seed"], a["m"], None)

    assert call(jump=0) == ERR_ARG
    assert call(jump=65536) == ERR_ARG
    assert call(m=-1) == ERR_ARG
    assert call(m=17) == ERR_ARG
    assert call(n=-1) == ERR_ARG
    assert call(W=-1) == ERR_ARG
    assert call(H=70000) == ERR_ARG
    assert call(W=65536) == ERR_ARG      # one past SAD_MAX_DIM (65535, the largest accepted)
    assert call(H=65536) == ERR_ARG
    assert call(rec=0) == ERR_ARG
    assert call(rec=0, W=0) == 0         # empty image: pointers are not needed
    assert call(rec=P + 8) == ERR_ALIGN
    assert call(b=P) == ERR_ARG          # in place
    assert call(b=P + 32) == ERR_ARG     # overlapping maps
    assert call(a=P + 4, b=Q) == ERR_ALIGN
    assert call(W=0) == 0                # empty image: no-op, nothing launched
    assert call(H=0, b=P) == 0           # empty: zero bytes cannot overlap
    assert call(cell=0) == ERR_ARG
    assert call(cell=-4) == ERR_ARG
    assert call(cell=65536) == ERR_ARG
    assert call(cell=0, W=0) == ERR_ARG  # the cell size is checked before the empty image
    # overlap is judged on the map's size: 16x16 pixels in cells of 4 -> 4x4 lists, 512 bytes
    assert call(cell=4, b=P + 480) == ERR_ARG
    assert call(fmt=2) == ERR_ARG        # unknown site format
    assert call(fmt=-1) == ERR_ARG
    assert call(fmt=1, rec=P + 8) == ERR_ALIGN
    assert call(scr=Q + 2) == ERR_ALIGN     # screen words need 4 bytes


def test_site_buffer_calls_reject_bad_arguments(L):
    f = L.sad_topk_propagate
    ok = dict(s=P, n=4, st=8, a=P, b=Q, W=16, H=16, jump=1, pidx=0, seed=0, m=4)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["s"], a["n"], a["st"], a["a"], a["b"], a["W"], a["H"], a["jump"], a["pidx"], a["seed"], a["m"],
                 None)

    assert call(n=9) == ERR_ARG          # n_slots > stride
    assert call(st=0) == ERR_ARG
    assert call(jump=0) == ERR_ARG
    assert call(m=17) == ERR_ARG
    assert call(s=0) == ERR_ARG
    assert call(b=P + 32) == ERR_ARG     # overlapping maps
    assert call(a=P + 4) == ERR_ALIGN
    assert call(s=P + 4, W=0) == 0       # the planes need only float alignment
    assert call(W=0) == 0
    assert call(H=65536) == ERR_ARG
    R, F = L.sad_render_fwd, L.sad_render_bwd
    assert R(P, 4, 8, P + 8, 16, 16, Q, None) == ERR_ALIGN
    assert R(P, 4, 8, 0, 16, 16, Q, None) == ERR_ARG
    assert R(P, 9, 8, P, 16, 16, Q, None) == ERR_ARG
    assert R(0, 4, 8, P, 16, 16, Q, None) == ERR_ARG
    assert R(P, 4, 8, P, 0, 16, Q, None) == 0
    assert R(P, 4, 8, P, 65536, 1, Q, None) == ERR_ARG
    assert F(P, 4, 8, P, 0, 16, 16, Q, None, None) == ERR_ARG     # target NULL
    assert F(P, 4, 8, P + 4, Q, 16, 16, Q, None, None) == ERR_ALIGN
    assert F(P, 4, 8, P, Q, 16, 16, Q + 2, None, None) == ERR_ALIGN  # grad planes: float alignment
    assert F(P, 4, 8, P, Q, 16, 16, 0, None, None) == ERR_ARG     # grad NULL
    assert F(P, 9, 8, P, Q, 16, 16, Q, None, None) == ERR_ARG
    assert F(P, 4, 8, P, Q, 1, 65536, Q, None, None) == ERR_ARG
    cfg = sad.AdamConfig().to_c(16, 16)
    A = L.sad_adam_step
    assert A(P, P, P, P, 4, 8, 0, 10, ctypes.byref(cfg), None) == ERR_ARG   # step 0
    assert A(P, P, P, P, 4, 8, 1, 0, ctypes.byref(cfg), None) == ERR_ARG   # no pixels
    assert A(P, P, P, P, 4, 8, 1, 10, None, None) == ERR_ARG
    assert A(P, P, P, 0, 4, 8, 1, 10, ctypes.byref(cfg), None) == ERR_ARG
    assert A(P, P, P, P, 9, 8, 1, 10, ctypes.byref(cfg), None) == ERR_ARG
    assert A(P, P, P, P, 0, 8, 1, 10, ctypes.byref(cfg), None) == 0        # no slots: no-op
    nobox = sad.AdamConfig().to_c(16, 16)
    nobox.x_max = 0.0
    assert A(P, P, P, P, 4, 8, 1, 10, ctypes.byref(nobox), None) == ERR_ARG  # no clamp box


def test_render_and_adam_reject_bad_arguments(L):
    assert L.sad_render_fwd_rec(P, 4, P + 8, 16, 16, 1, Q, None) == ERR_ALIGN
    assert L.sad_render_fwd_rec(P + 8, 4, P, 16, 16, 1, Q, None) == ERR_ALIGN
    assert L.sad_render_fwd_rec(P, 4, 0, 16, 16, 1, Q, None) == ERR_ARG
    assert L.sad_render_fwd_rec(P, -1, P, 16, 16, 1, Q, None) == ERR_ARG
    assert L.sad_render_fwd_rec(0, 4, P, 16, 16, 1, Q, None) == ERR_ARG
    assert L.sad_render_fwd_rec(P, 4, P, 0, 16, 1, Q, None) == 0
    assert L.sad_render_fwd_rec(P, 4, P, 16, 16, 0, Q, None) == ERR_ARG  # cell 0
    assert L.sad_render_fwd_rec(P, 4, P, 65536, 1, 1, Q, None) == ERR_ARG  # beyond SAD_MAX_DIM
    B = L.sad_render_bwd_rec
    assert B(P, 4, P, Q, 1, 65536, 1, Q, None, None, None) == ERR_ARG
    assert B(P, 4, P, 0, 16, 16, 1, Q, None, None, None) == ERR_ARG  # target NULL
    assert B(P, 4, P + 4, Q, 16, 16, 1, Q, None, None, None) == ERR_ALIGN
    assert B(P, 4, P, Q, 16, 16, 1, Q + 4, None, None, None) == ERR_ALIGN  # grad records
    assert B(P, 4, P, Q, 16, 16, 0, Q, None, None, None) == ERR_ARG  # cell 0
    X = L.sad_topk_exact_at
    assert X(P, 0, 4, P, -1, 16, 16, 1, Q, None) == ERR_ARG
    assert X(P, 0, 4, P + 2, 4, 16, 16, 1, Q, None) == ERR_ALIGN
    assert X(P, 0, 4, P, 4, 16, 16, 1, Q + 4, None) == ERR_ALIGN
    assert X(P, 0, 4, P, 0, 16, 16, 1, Q, None) == 0                # no entries: no-op
    assert X(P, 2, 4, P, 4, 16, 16, 1, Q, None) == ERR_ARG          # unknown site format
    C = L.sad_site_screen
    assert C(P, 4, 8, 16, 16, Q + 2, None) == ERR_ALIGN
    assert C(P, 9, 8, 16, 16, Q, None) == ERR_ARG
    assert C(P, 4, 8, 0, 16, Q, None) == ERR_ARG                    # no image: no cell size
    assert C(0, 4, 8, 16, 16, Q, None) == ERR_ARG
    assert C(0, 0, 8, 16, 16, 0, None) == 0                         # no slots: no-op
    S = L.sad_apply_seeds
    assert S(P, 16, 16, 1, P, -1, None) == ERR_ARG
    assert S(P, 16, 16, 0, P, 4, None) == ERR_ARG
    assert S(P + 4, 16, 16, 1, P, 4, None) == ERR_ALIGN
    assert S(P, 16, 16, 1, P + 4, 4, None) == ERR_ALIGN
    assert S(0, 16, 16, 1, P, 4, None) == ERR_ARG
    assert S(P, 16, 16, 1, P, 0, None) == 0                         # no pairs: no-op
    assert L.sad_topk_exact(P, 0, 4, P + 4, 16, 16, 1, None) == ERR_ALIGN
    assert L.sad_topk_exact(P, 0, -1, P, 16, 16, 1, None) == ERR_ARG
    assert L.sad_topk_exact(P, 0, 4, P, 16, 16, 0, None) == ERR_ARG
    assert L.sad_topk_exact(P, 5, 4, P, 16, 16, 1, None) == ERR_ARG  # unknown site format
    assert L.sad_pack_sites(P, 4, 8, P + 4, None) == ERR_ALIGN
    assert L.sad_pack_sites(P, 9, 8, P, None) == ERR_ARG
    assert L.sad_pack_sites(0, 4, 8, P, None) == ERR_ARG
    assert L.sad_pack_sites(P, 4, 8, 0, None) == ERR_ARG
    assert L.sad_pack_sites(0, 0, 8, 0, None) == 0  # no slots: no-op
    assert L.sad_site_records(P, 4, 8, P + 4, None) == ERR_ALIGN
    assert L.sad_site_records(P, 9, 8, P, None) == ERR_ARG
    assert L.sad_site_records(0, 4, 8, P, None) == ERR_ARG
    assert L.sad_site_records(0, 0, 8, 0, None) == 0  # no slots: no-op
    cfg = sad.AdamConfig().to_c(4, 4)
    A = L.sad_adam_step_rec
    assert A(P, P, P, P, P, None, None, 4, 8, 0, 10, ctypes.byref(cfg), None) == ERR_ARG   # step 0
    assert A(P, P, P, P, P, None, None, 4, 8, 1, 0, ctypes.byref(cfg), None) == ERR_ARG   # no pixels
    assert A(P, P, P, P, P, None, None, 4, 8, 1, 10, None, None) == ERR_ARG
    assert A(P, P, P, P + 4, P, None, None, 4, 8, 1, 10, ctypes.byref(cfg), None) == ERR_ALIGN
    assert A(P, P, P, P, P + 4, None, None, 4, 8, 1, 10, ctypes.byref(cfg), None) == ERR_ALIGN
    bad = sad.AdamConfig(beta1=1.0).to_c(4, 4)
    assert A(P, P, P, P, P, None, None, 4, 8, 1, 10, ctypes.byref(bad), None) == ERR_ARG
    assert A(P, P, P, P, None, None, None, 0, 8, 1, 10, ctypes.byref(cfg), None) == 0  # no slots: no-op
    assert A(P, P, P, P, P, P + 4, None, 4, 8, 1, 10, ctypes.byref(cfg), None) == ERR_ALIGN  # packed
    assert A(P, P, P, P, P, None, Q + 2, 4, 8, 1, 10, ctypes.byref(cfg), None) == ERR_ALIGN  # screen


def test_jfa_entry_points_reject_bad_arguments(L):
    S, J = L.sad_jfa_seed, L.sad_jfa_pass
    assert S(P, 0, -1, P, 16, 16, 1, None) == ERR_ARG
    assert S(0, 0, 4, P, 16, 16, 1, None) == ERR_ARG
    assert S(P, 0, 4, 0, 16, 16, 1, None) == ERR_ARG
    assert S(P, 0, 4, P + 4, 16, 16, 1, None) == ERR_ALIGN
    assert S(P + 8, 0, 4, P, 16, 16, 1, None) == ERR_ALIGN
    assert S(P, 0, 4, P, 70000, 16, 1, None) == ERR_ARG
    assert S(P, 0, 4, P, 0, 16, 1, None) == 0                      # empty image: no-op
    assert J(P, 0, 4, P, Q, 16, 16, 1, 0, None) == ERR_ARG         # step 0
    assert J(P, 0, 4, P, Q, 16, 16, 1, 65536, None) == ERR_ARG
    assert J(P, 0, 4, P, P + 32, 16, 16, 1, 1, None) == ERR_ARG     # overlapping maps
    assert J(P, 0, 4, P + 4, Q, 16, 16, 1, 1, None) == ERR_ALIGN
    assert J(P, 0, -1, P, Q, 16, 16, 1, 1, None) == ERR_ARG
    assert J(P, 0, 4, P, Q, 16, 0, 1, 1, None) == 0
    assert S(P, 0, 4, P, 16, 16, 0, None) == ERR_ARG            # cell 0
    assert J(P, 0, 4, P, Q, 16, 16, 0, 1, None) == ERR_ARG
    assert J(P, 0, 4, P, P + 256, 16, 16, 2, 1, None) == ERR_ARG  # 8x8 lists of 32 bytes overlap
    assert S(P, 3, 4, P, 16, 16, 1, None) == ERR_ARG         # unknown site format
    assert J(P, 3, 4, P, Q, 16, 16, 1, 1, None) == ERR_ARG


def test_densify_entry_points_reject_bad_arguments(L):
    D = L.sad_densify_stats
    assert D(P, -1, P, Q, 16, 16, 1, Q, None) == ERR_ARG
    assert D(P, 4, 0, Q, 16, 16, 1, Q, None) == ERR_ARG        # cand NULL
    assert D(P, 4, P, 0, 16, 16, 1, Q, None) == ERR_ARG        # target NULL
    assert D(P, 4, P, Q, 16, 16, 1, 0, None) == ERR_ARG        # stats NULL
    assert D(P, 4, P + 4, Q, 16, 16, 1, Q, None) == ERR_ALIGN
    assert D(P, 4, P, Q, 16, 16, 1, Q + 4, None) == ERR_ALIGN
    assert D(P, 4, P, Q, 0, 16, 1, Q, None) == 0               # empty image: no-op
    assert D(P, 4, P, Q, 16, 70000, 1, Q, None) == ERR_ARG
    assert D(P, 4, P, Q, 16, 16, 0, Q, None) == ERR_ARG     # cell 0
    cfg = sad.BudgetConfig().to_c()
    n = ctypes.c_int(4)
    F = L.sad_densify_prune_stats
    assert F(None, P, P, 8, 8, ctypes.byref(n), P, P, P, 4, 4, 1, P, ctypes.byref(cfg), None, None, None, 0, None) == ERR_ARG
    assert F(P, P, P, 8, 8, None, P, P, P, 4, 4, 1, P, ctypes.byref(cfg), None, None, None, 0, None) == ERR_ARG
    assert F(P, P, P, 8, 8, ctypes.byref(n), P, P, P, 4, 4, 1, P, None, None, None, None, 0, None) == ERR_ARG
    assert F(P, P, P, 8, 3, ctypes.byref(n), P, P, P, 4, 4, 1, P, ctypes.byref(cfg), None, None, None, 0, None) == ERR_ARG
    assert F(P, P, P, 8, 9, ctypes.byref(n), P, P, P, 4, 4, 1, P, ctypes.byref(cfg), None, None, None, 0, None) == ERR_ARG
    assert F(P, P, P, 8, 8, ctypes.byref(n), P, P, P, 0, 4, 1, P, ctypes.byref(cfg), None, None, None, 0, None) == ERR_ARG
    assert F(P, P, P, 8, 8, ctypes.byref(n), P, P, P, 4, 4, 0, P, ctypes.byref(cfg), None, None, None, 0, None) == ERR_ARG
    assert n.value == 4
    G = L.sad_densify_prune
    seed = ctypes.c_uint64(7)
    assert G(None, P, P, P, ctypes.byref(n), 8, 8, P, 4, 4, P, ctypes.byref(cfg), seed) == ERR_ARG
    assert G(P, P, P, P, None, 8, 8, P, 4, 4, P, ctypes.byref(cfg), seed) == ERR_ARG
    assert G(P, P, P, P, ctypes.byref(n), 8, 8, None, 4, 4, P, ctypes.byref(cfg), seed) == ERR_ARG  # cand
    assert G(P, P, P, P, ctypes.byref(n), 3, 8, P, 4, 4, P, ctypes.byref(cfg), seed) == ERR_ARG  # capacity < n
    assert G(P, P, P, P, ctypes.byref(n), 9, 8, P, 4, 4, P, ctypes.byref(cfg), seed) == ERR_ARG  # capacity > stride
    assert G(P, P, P, P, ctypes.byref(n), 8, 8, P, 0, 4, P, ctypes.byref(cfg), seed) == ERR_ARG
    assert G(P, P, P, P, ctypes.byref(n), 8, 8, P, 4, 4, P, None, seed) == ERR_ARG
    assert n.value == 4


def test_eval_entry_points_reject_bad_arguments(L):
    E, D, Qy = L.sad_eval_encode, L.sad_eval_decode, L.sad_eval_query
    assert E(P, 4, 8, 16, 16, P + 4, Q, None) == ERR_ALIGN     # words
    assert E(P, 4, 8, 16, 16, P, Q + 4, None) == ERR_ALIGN     # header
    assert E(P, 4, 8, 0, 16, P, Q, None) == ERR_ARG            # W = 0: no position scale
    assert E(P, 9, 8, 16, 16, P, Q, None) == ERR_ARG           # n_slots > stride
    assert E(P, 4, 8, 16, 16, P, 0, None) == ERR_ARG           # header NULL
    assert E(0, 4, 8, 16, 16, P, Q, None) == ERR_ARG
    assert D(P + 4, Q, 4, 16, 16, P, 8, None) == ERR_ALIGN
    assert D(P, Q, 9, 16, 16, P, 8, None) == ERR_ARG
    assert D(P, Q, 0, 16, 16, 0, 8, None) == 0                 # no slots: no-op
    assert D(0, Q, 4, 16, 16, P, 8, None) == ERR_ARG
    assert Qy(P, Q, 4, P, 16, 16, 1, P, 0, Q, None) == 0       # no points: no-op
    assert Qy(P, Q, 4, P, 16, 16, 0, P, 5, Q, None) == ERR_ARG  # cell 0
    assert Qy(P, Q, 4, P, 16, 16, 1, P, -1, Q, None) == ERR_ARG
    assert Qy(P, Q, 4, P, 16, 16, 1, P + 4, 5, Q, None) == ERR_ALIGN  # points need 8 bytes
    assert Qy(P, Q, 4, P + 8, 16, 16, 1, P, 5, Q, None) == ERR_ALIGN  # cand needs 16
    assert Qy(P, Q, 4, P, 16, 16, 1, P, 2 ** 31, Q, None) == ERR_ARG
    assert Qy(P, Q, 4, P, 16, 16, 1, 0, 5, Q, None) == ERR_ARG


def test_python_binding_refuses_cpu_tensors():
    import torch
    s = torch.zeros((10, 4))
    with pytest.raises(ValueError):
        sad.render_fwd_rec(torch.zeros((4, 16)), 4, torch.zeros((2, 2, 8), dtype=torch.int32), 2, 2,
                           torch.zeros((2, 2, 3)))
    with pytest.raises(ValueError):
        sad.render_fwd(torch.zeros((10, 4)), 4, torch.zeros((2, 2, 8), dtype=torch.int32), 2, 2,
                       torch.zeros((2, 2, 3)))
    with pytest.raises(ValueError):
        sad.site_records(s, 4, torch.zeros((4, 16)))


def test_jump_schedule():
    assert sad.jump_schedule(768, 512, 12) == [512, 256, 128, 64, 32, 16, 8, 4, 2, 1, 1, 1]
    assert sad.jump_schedule(4096, 4096, 13)[:12] == [2048 >> i for i in range(12)]
    assert sad.jump_schedule(1, 1, 3) == [1, 1, 1]
    # on a map of 4x4-pixel cells the schedule counts map entries (192 x 128)
    assert sad.jump_schedule(768, 512, 9, cell=4) == [128, 64, 32, 16, 8, 4, 2, 1, 1]
    assert sad.jfa_steps(768, 512, cell=4) == [128, 64, 32, 16, 8, 4, 2, 1]
    assert sad.map_shape(77, 45, 4) == (12, 20, 8)
    with pytest.raises(ValueError):
        sad.map_shape(16, 16, 0)
