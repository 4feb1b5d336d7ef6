"""soft_voronoi_render_amd -- MI355X (gfx950) hot path of Soft Anisotropic Diagrams (SAD).

The compute lives in ``libsad.so`` (hand-written HIP kernels behind the C ABI of
``include/sad.h``).  This module is argument marshalling only: it takes torch
tensors that already live on the GPU, checks dtype/shape/device, and passes raw
device pointers and the caller's HIP stream to the library.  There is no CPU
fallback: if the library is not built, or a tensor is not on a GPU, the call
raises.

Layouts (see include/sad.h): sites float32 [10][stride], candidate map uint32
[H][W][8] (torch int32 storage reinterpreted), images float32 [H][W][3], Adam
moments float32 [10][stride].  Gradients: float32 [11][stride] planes for the
site-buffer calls (topk_propagate, render_fwd, render_bwd, adam_step,
densify_prune), float32 [stride][16] records (10 gradients, the removal delta,
5 unused words) for the cached calls (the *_rec names), which read the derived
site records or packed words instead of the planes.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libsad.so")
SOURCES = [os.path.join(HERE, "csrc", "sad_kernels.hip"), os.path.join(HERE, "csrc", "sad_budget.cpp")]
INCLUDE = os.path.join(ROOT, "include")

K = 8
INVALID = 0xFFFFFFFF
NPARAM = 10
NACC = 11
GRAD_LD = 16
REC_LD = 16
STAT_LD = 8
LOSS_SLOTS = 64
MAX_INJECT = 16
PACK_LD = 4
SEL_REC64, SEL_PACKED16 = 0, 1

SAD_OK, SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE, SAD_ERR_CAPACITY, SAD_ERR_UNIMPLEMENTED = 0, -1, -2, -3, -4, -5
STATUS = {0: "ok", -1: "invalid argument", -2: "misaligned pointer", -3: "HIP launch failed",
          -4: "capacity exceeded", -5: "not implemented"}

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-munsafe-fp-atomics",
    # packed FP32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


class SadError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn}: {STATUS.get(rc, 'unknown status')} ({rc})")
        self.rc = rc


def build(verbose: bool = False) -> str:
    """Compile libsad.so for gfx950 in-tree with hipcc."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", INCLUDE, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB_PATH)
    global _lib
    _lib = None
    return LIB_PATH


class BudgetCfg(ctypes.Structure):
    _fields_ = [("split_frac", ctypes.c_float), ("prune_frac", ctypes.c_float), ("alpha", ctypes.c_float),
                ("min_mass", ctypes.c_float), ("shrink", ctypes.c_float)]


class AdamCfg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float * NPARAM), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("x_max", ctypes.c_float), ("y_max", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsad.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (soft_voronoi_render_amd.build()); "
                               "there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p
        L.sad_abi_version.restype = i32
        L.sad_abi_version.argtypes = []
        L.sad_status_string.restype = ctypes.c_char_p
        L.sad_status_string.argtypes = [i32]
        L.sad_site_records.restype = i32
        L.sad_site_records.argtypes = [fp, i32, i32, fp, vp]
        L.sad_topk_propagate.restype = i32
        L.sad_topk_propagate.argtypes = [fp, i32, i32, vp, vp, i32, i32, i32, u32, u32, i32, vp]
        L.sad_topk_propagate_rec.restype = i32
        L.sad_topk_propagate_rec.argtypes = [vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, u32, u32, i32, vp]
        L.sad_site_screen.restype = i32
        L.sad_site_screen.argtypes = [fp, i32, i32, i32, i32, vp, vp]
        L.sad_eval_encode.restype = i32
        L.sad_eval_encode.argtypes = [fp, i32, i32, i32, i32, vp, fp, vp]
        L.sad_eval_decode.restype = i32
        L.sad_eval_decode.argtypes = [vp, fp, i32, i32, i32, fp, i32, vp]
        L.sad_eval_query.restype = i32
        L.sad_eval_query.argtypes = [vp, fp, i32, vp, i32, i32, i32, fp, ctypes.c_int64, fp, vp]
        L.sad_pack_sites.restype = i32
        L.sad_pack_sites.argtypes = [fp, i32, i32, vp, vp]
        L.sad_topk_exact.restype = i32
        L.sad_topk_exact.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp]
        L.sad_topk_exact_at.restype = i32
        L.sad_topk_exact_at.argtypes = [vp, i32, i32, vp, i32, i32, i32, i32, vp, vp]
        L.sad_render_fwd.restype = i32
        L.sad_render_fwd.argtypes = [fp, i32, i32, vp, i32, i32, fp, vp]
        L.sad_render_fwd_rec.restype = i32
        L.sad_render_fwd_rec.argtypes = [fp, i32, vp, i32, i32, i32, fp, vp]
        L.sad_render_bwd.restype = i32
        L.sad_render_bwd.argtypes = [fp, i32, i32, vp, fp, i32, i32, fp, fp, vp]
        L.sad_render_bwd_rec.restype = i32
        L.sad_render_bwd_rec.argtypes = [fp, i32, vp, fp, i32, i32, i32, fp, fp, fp, vp]
        L.sad_apply_seeds.restype = i32
        L.sad_apply_seeds.argtypes = [vp, i32, i32, i32, vp, ctypes.c_long, vp]
        L.sad_jfa_seed.restype = i32
        L.sad_jfa_seed.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp]
        L.sad_jfa_pass.restype = i32
        L.sad_jfa_pass.argtypes = [vp, i32, i32, vp, vp, i32, i32, i32, i32, vp]
        L.sad_densify_stats.restype = i32
        L.sad_densify_stats.argtypes = [fp, i32, vp, fp, i32, i32, i32, fp, vp]
        ip = ctypes.POINTER(ctypes.c_int)
        L.sad_densify_prune_stats.restype = i32
        L.sad_densify_prune_stats.argtypes = [fp, fp, fp, i32, i32, ip, fp, fp, vp, i32, i32, i32, fp,
                                              ctypes.POINTER(BudgetCfg), ip, ip, vp, ctypes.c_long,
                                              ctypes.POINTER(ctypes.c_long)]
        L.sad_densify_prune.restype = i32
        L.sad_densify_prune.argtypes = [fp, fp, fp, fp, ip, i32, i32, vp, i32, i32, fp, ctypes.POINTER(BudgetCfg),
                                        ctypes.c_uint64]
        L.sad_adam_step.restype = i32
        L.sad_adam_step.argtypes = [fp, fp, fp, fp, i32, i32, i32, i32, ctypes.POINTER(AdamCfg), vp]
        L.sad_adam_step_rec.restype = i32
        L.sad_adam_step_rec.argtypes = [fp, fp, fp, fp, fp, vp, vp, i32, i32, i32, i32, ctypes.POINTER(AdamCfg), vp]
        _lib = L
    return _lib


EXPORTED = ("sad_abi_version", "sad_status_string",
            # the iteration on the site buffer
            "sad_topk_propagate", "sad_render_fwd", "sad_render_bwd", "sad_adam_step", "sad_densify_prune",
            # the iteration on derived caches
            "sad_site_records", "sad_pack_sites", "sad_site_screen", "sad_topk_propagate_rec", "sad_render_fwd_rec",
            "sad_render_bwd_rec", "sad_adam_step_rec", "sad_densify_stats", "sad_densify_prune_stats",
            "sad_apply_seeds",
            # candidate-map tools, evaluation format
            "sad_jfa_seed", "sad_jfa_pass", "sad_topk_exact", "sad_topk_exact_at", "sad_eval_encode",
            "sad_eval_decode", "sad_eval_query")


# --------------------------------------------------------------- marshalling
def _dev(t: torch.Tensor, name: str, dtypes, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU fallback)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise SadError(fn, rc)


_F32 = (torch.float32,)
_U32 = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _sites(sites: torch.Tensor, n_slots: int):
    if sites.dim() != 2 or sites.shape[0] != NPARAM:
        raise ValueError("sites must be float32 [10][stride]")
    ptr = _dev(sites, "sites", _F32)
    stride = sites.shape[1]
    if not 0 <= n_slots <= stride:
        raise ValueError("need 0 <= n_slots <= stride")
    return ptr, stride


def _rec(rec: torch.Tensor, n_slots: int) -> int:
    if rec.dim() != 2 or rec.shape[1] != REC_LD or rec.shape[0] < n_slots:
        raise ValueError("rec must be float32 [>= n_slots][16]")
    return _dev(rec, "rec", _F32)


def new_records(capacity: int, device="cuda") -> torch.Tensor:
    """Storage for the per-site records, float32 [capacity][16]."""
    return torch.zeros((max(capacity, 1), REC_LD), dtype=torch.float32, device=device)


def new_packed(capacity: int, device="cuda") -> torch.Tensor:
    """Storage for the packed candidate-site buffer, uint32 [capacity][4] held as int32."""
    return torch.zeros((max(capacity, 1), PACK_LD), dtype=torch.int32, device=device)


def _sel(sel: torch.Tensor, n_slots: int):
    """(pointer, format) of the site buffer a selection entry point reads: the
    records (float32 [>= n][16]) or the packed buffer (int32 [>= n][4])."""
    if sel.dim() == 2 and sel.dtype == torch.float32 and sel.shape[1] == REC_LD and sel.shape[0] >= n_slots:
        return _dev(sel, "rec", _F32), SEL_REC64
    if sel.dim() == 2 and sel.dtype in _U32 and sel.shape[1] == PACK_LD and sel.shape[0] >= n_slots:
        return _dev(sel, "packed", _U32), SEL_PACKED16
    raise ValueError("selection sites must be records float32 [>= n_slots][16] or packed int32 [>= n_slots][4]")


def pack_sites(sites, n_slots, packed, stream=None):
    """Writes the packed candidate-site words of slots [0, n_slots) (see sad_pack_sites)."""
    sp, stride = _sites(sites, n_slots)
    if packed.dim() != 2 or packed.shape[1] != PACK_LD or packed.shape[0] < n_slots:
        raise ValueError("packed must be int32 [>= n_slots][4]")
    pk = _dev(packed, "packed", _U32)
    _check("sad_pack_sites", lib().sad_pack_sites(sp, n_slots, stride, pk, _stream(stream)))


def site_records(sites, n_slots, rec, stream=None):
    """Writes the site records of slots [0, n_slots) (see sad_site_records)."""
    sp, stride = _sites(sites, n_slots)
    r = _rec(rec, n_slots)
    _check("sad_site_records", lib().sad_site_records(sp, n_slots, stride, r, _stream(stream)))


def new_screen(capacity: int, device="cuda") -> torch.Tensor:
    """Storage for the candidate screen, uint32 [capacity] held as int32."""
    return torch.zeros(max(capacity, 1), dtype=torch.int32, device=device)


def _scr(scr, n_slots):
    if scr is None:
        return None
    if scr.dim() != 1 or scr.shape[0] < n_slots:
        raise ValueError("scr must be int32 [>= n_slots]")
    return _dev(scr, "scr", _U32)


def site_screen(sites, n_slots, W, H, scr, stream=None):
    """Writes the candidate-screen words of slots [0, n_slots) for a W x H image
    (see sad_site_screen)."""
    sp, stride = _sites(sites, n_slots)
    _check("sad_site_screen", lib().sad_site_screen(sp, n_slots, stride, W, H, _scr(scr, n_slots),
                                                    _stream(stream)))


def map_shape(W: int, H: int, cell: int = 1) -> tuple:
    """Shape of the candidate map of a W x H image with cells of `cell` x `cell`
    pixels: (ceil(H / cell), ceil(W / cell), 8)."""
    if cell < 1:
        raise ValueError("cell must be >= 1")
    return (-(-H // cell), -(-W // cell), K)


def topk_propagate(sites, n_slots, cand_in, cand_out, W, H, jump, pass_index, seed, n_inject, stream=None):
    """One propagation pass of the per-pixel map, reading the site planes:
    cand_in -> cand_out (see sad_topk_propagate)."""
    sp, stride = _sites(sites, n_slots)
    a = _dev(cand_in, "cand_in", _U32, map_shape(W, H))
    b = _dev(cand_out, "cand_out", _U32, map_shape(W, H))
    _check("sad_topk_propagate", lib().sad_topk_propagate(sp, n_slots, stride, a, b, W, H, jump,
                                                          pass_index & 0xFFFFFFFF, seed & 0xFFFFFFFF, n_inject,
                                                          _stream(stream)))


def topk_propagate_rec(rec, n_slots, cand_in, cand_out, W, H, jump, pass_index, seed, n_inject, stream=None, cell=1,
                       scr=None):
    """One propagation pass: cand_in -> cand_out (see sad_topk_propagate_rec).
    `rec` is the record buffer or the packed candidate-site buffer; `scr` the
    candidate screen or None."""
    g, fmt = _sel(rec, n_slots)
    a = _dev(cand_in, "cand_in", _U32, map_shape(W, H, cell))
    b = _dev(cand_out, "cand_out", _U32, map_shape(W, H, cell))
    _check("sad_topk_propagate_rec", lib().sad_topk_propagate_rec(g, fmt, _scr(scr, n_slots), n_slots, a, b, W, H,
                                                                  cell, jump,
                                                                  pass_index & 0xFFFFFFFF, seed & 0xFFFFFFFF,
                                                                  n_inject, _stream(stream)))


def jfa_seed(rec, n_slots, cand, W, H, stream=None, cell=1):
    """Seed pass of the jump-flood prepass (see sad_jfa_seed)."""
    g, fmt = _sel(rec, n_slots)
    c = _dev(cand, "cand", _U32, map_shape(W, H, cell))
    _check("sad_jfa_seed", lib().sad_jfa_seed(g, fmt, n_slots, c, W, H, cell, _stream(stream)))


def jfa_pass(rec, n_slots, cand_in, cand_out, W, H, step, stream=None, cell=1):
    """One flood pass of the jump-flood prepass: cand_in -> cand_out (see sad_jfa_pass)."""
    g, fmt = _sel(rec, n_slots)
    a = _dev(cand_in, "cand_in", _U32, map_shape(W, H, cell))
    b = _dev(cand_out, "cand_out", _U32, map_shape(W, H, cell))
    _check("sad_jfa_pass", lib().sad_jfa_pass(g, fmt, n_slots, a, b, W, H, cell, step, _stream(stream)))


def jfa_steps(W: int, H: int, cell: int = 1) -> list:
    """The prepass's flood steps B/2, ..., 1 with B = 2^ceil(log2 max(Wm, Hm)),
    counted in map entries."""
    Hm, Wm, _ = map_shape(W, H, cell)
    B = 1 << max(0, (max(Wm, Hm) - 1).bit_length())
    out, k = [], B // 2
    while k >= 1:
        out.append(k)
        k //= 2
    return out


def jfa_prepass(rec, n_slots, a, b, W, H, stream=None, cell=1):
    """Seed pass into `a`, then the flood passes ping-ponging between `a` and `b`;
    returns the map that holds the result (four closest per entry)."""
    jfa_seed(rec, n_slots, a, W, H, stream, cell)
    for k in jfa_steps(W, H, cell):
        jfa_pass(rec, n_slots, a, b, W, H, k, stream, cell)
        a, b = b, a
    return a


def topk_exact(rec, n_slots, cand_out, W, H, stream=None, cell=1):
    """Brute-force exact top-K map (see sad_topk_exact)."""
    g, fmt = _sel(rec, n_slots)
    b = _dev(cand_out, "cand_out", _U32, map_shape(W, H, cell))
    _check("sad_topk_exact", lib().sad_topk_exact(g, fmt, n_slots, b, W, H, cell, _stream(stream)))


def topk_exact_at(rec, n_slots, entries, W, H, out, stream=None, cell=1):
    """Exact top-K lists of the map entries `entries` (int32 [n], indices
    row*Wm + col) into out (int32 [n][8]) (see sad_topk_exact_at)."""
    g, fmt = _sel(rec, n_slots)
    if entries.dim() != 1:
        raise ValueError("entries must be int32 [n]")
    n = entries.shape[0]
    e = _dev(entries, "entries", _U32)
    o = _dev(out, "out", _U32, (n, K))
    _check("sad_topk_exact_at", lib().sad_topk_exact_at(g, fmt, n_slots, e, n, W, H, cell, o, _stream(stream)))


def render_fwd(sites, n_slots, cand, W, H, out_rgb, stream=None):
    """Temperature-softmax render of each pixel's list from the site planes (see
    sad_render_fwd)."""
    sp, stride = _sites(sites, n_slots)
    c = _dev(cand, "cand", _U32, map_shape(W, H))
    o = _dev(out_rgb, "out_rgb", _F32, (H, W, 3))
    _check("sad_render_fwd", lib().sad_render_fwd(sp, n_slots, stride, c, W, H, o, _stream(stream)))


def render_fwd_rec(rec, n_slots, cand, W, H, out_rgb, stream=None, cell=1):
    """Temperature-softmax render of each pixel's list (see sad_render_fwd_rec)."""
    r = _rec(rec, n_slots)
    c = _dev(cand, "cand", _U32, map_shape(W, H, cell))
    o = _dev(out_rgb, "out_rgb", _F32, (H, W, 3))
    _check("sad_render_fwd_rec", lib().sad_render_fwd_rec(r, n_slots, c, W, H, cell, o, _stream(stream)))


def new_loss(device) -> torch.Tensor:
    """Zeroed loss accumulator for render_bwd: LOSS_SLOTS partial sums whose sum
    is the loss."""
    return torch.zeros(LOSS_SLOTS, dtype=torch.float32, device=device)


def render_bwd(sites, n_slots, cand, target, W, H, grad, loss_sum=None, stream=None):
    """Gradients of the squared error from the site planes, accumulated into the
    gradient planes grad float32 [11][stride]; loss_sum, a one-element float32
    tensor, receives the summed squared error (see sad_render_bwd)."""
    sp, stride = _sites(sites, n_slots)
    c = _dev(cand, "cand", _U32, map_shape(W, H))
    t = _dev(target, "target", _F32, (H, W, 3))
    g = _dev(grad, "grad", _F32, (NACC, stride))
    if loss_sum is not None and loss_sum.numel() != 1:
        raise ValueError("loss_sum must hold one float32")
    ls = _dev(loss_sum, "loss_sum", _F32) if loss_sum is not None else None
    _check("sad_render_bwd", lib().sad_render_bwd(sp, n_slots, stride, c, t, W, H, g, ls, _stream(stream)))


def render_bwd_rec(rec, n_slots, cand, target, W, H, grad, loss_sum=None, out_rgb=None, stream=None, cell=1):
    """Gradients of the squared error, accumulated into the gradient records;
    optionally also the rendered image (see sad_render_bwd_rec)."""
    r = _rec(rec, n_slots)
    c = _dev(cand, "cand", _U32, map_shape(W, H, cell))
    t = _dev(target, "target", _F32, (H, W, 3))
    if grad.dim() != 2 or grad.shape[1] != GRAD_LD or grad.shape[0] < n_slots:
        raise ValueError("grad must be float32 [>= n_slots][16]")
    g = _dev(grad, "grad", _F32)
    if loss_sum is not None and loss_sum.numel() != LOSS_SLOTS:
        raise ValueError(f"loss_sum must hold {LOSS_SLOTS} partial sums (see new_loss)")
    ls = _dev(loss_sum, "loss_sum", _F32) if loss_sum is not None else None
    o = _dev(out_rgb, "out_rgb", _F32, (H, W, 3)) if out_rgb is not None else None
    _check("sad_render_bwd_rec", lib().sad_render_bwd_rec(r, n_slots, c, t, W, H, cell, g, ls, o,
                                                          _stream(stream)))


@dataclasses.dataclass
class AdamConfig:
    """Adam settings.  The pages do not reproduce their learning rates; these
    defaults (px units for x, y, r) are ours."""
    lr: tuple = (0.1, 0.1, 0.02, 0.05, 0.01, 0.01, 0.01, 0.02, 0.02, 0.02)
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8

    def to_c(self, W: int, H: int) -> AdamCfg:
        """The C struct, with positions clamped to the W x H image."""
        c = AdamCfg()
        for j in range(NPARAM):
            c.lr[j] = float(self.lr[j])
        c.beta1, c.beta2, c.eps = self.beta1, self.beta2, self.eps
        c.x_max, c.y_max = float(W), float(H)
        return c


def _adam_cfg(cfg, W, H) -> AdamCfg:
    if isinstance(cfg, AdamCfg):
        return cfg
    return (cfg if cfg is not None else AdamConfig()).to_c(W, H)


def adam_step(sites, m, v, grad, n_slots, step, n_pixels, W, H, cfg: AdamConfig | AdamCfg | None = None,
              stream=None):
    """Adam on the site planes with gradient planes float32 [11][stride] (see
    sad_adam_step); positions are clamped to the W x H image."""
    sp, stride = _sites(sites, n_slots)
    mp = _dev(m, "m", _F32, (NPARAM, stride))
    vp = _dev(v, "v", _F32, (NPARAM, stride))
    g = _dev(grad, "grad", _F32, (NACC, stride))
    c = _adam_cfg(cfg, W, H)
    _check("sad_adam_step", lib().sad_adam_step(sp, mp, vp, g, n_slots, stride, step, n_pixels, ctypes.byref(c),
                                                _stream(stream)))


def adam_step_rec(sites, m, v, grad, n_slots, step, n_pixels, W, H, cfg: AdamConfig | AdamCfg | None = None,
                  rec=None, stream=None, packed=None, scr=None):
    """Adam on gradient records float32 [stride][16], refreshing the records,
    packed words and screen words if given (see sad_adam_step_rec)."""
    sp, stride = _sites(sites, n_slots)
    mp = _dev(m, "m", _F32, (NPARAM, stride))
    vp = _dev(v, "v", _F32, (NPARAM, stride))
    g = _dev(grad, "grad", _F32, (stride, GRAD_LD))
    gp = _rec(rec, n_slots) if rec is not None else None
    pk = None
    if packed is not None:
        if packed.dim() != 2 or packed.shape[1] != PACK_LD or packed.shape[0] < n_slots:
            raise ValueError("packed must be int32 [>= n_slots][4]")
        pk = _dev(packed, "packed", _U32)
    c = _adam_cfg(cfg, W, H)
    _check("sad_adam_step_rec", lib().sad_adam_step_rec(sp, mp, vp, g, gp, pk, _scr(scr, n_slots), n_slots, stride,
                                                        step, n_pixels, ctypes.byref(c), _stream(stream)))


def densify_stats(rec, n_slots, cand, target, W, H, stats, stream=None, cell=1):
    """Per-site mass, energy and error-weighted moments, accumulated into stats
    [>= n_slots][8] (see sad_densify_stats)."""
    r = _rec(rec, n_slots)
    c = _dev(cand, "cand", _U32, map_shape(W, H, cell))
    t = _dev(target, "target", _F32, (H, W, 3))
    if stats.dim() != 2 or stats.shape[1] != STAT_LD or stats.shape[0] < n_slots:
        raise ValueError("stats must be float32 [>= n_slots][8]")
    st = _dev(stats, "stats", _F32)
    _check("sad_densify_stats", lib().sad_densify_stats(r, n_slots, c, t, W, H, cell, st, _stream(stream)))


@dataclasses.dataclass
class BudgetConfig:
    """Budget-control settings (ours: the pages do not give their constants)."""
    split_frac: float = 0.05
    prune_frac: float = 0.05
    alpha: float = 0.5
    min_mass: float = 1.0
    shrink: float = 0.85

    def to_c(self) -> BudgetCfg:
        return BudgetCfg(self.split_frac, self.prune_frac, self.alpha, self.min_mass, self.shrink)


def densify_prune(sites, m, v, removal, n_slots, capacity, cand, W, H, target, cfg: BudgetConfig | None = None,
                  seed: int = 0):
    """Host-side budget control from the site buffer, on numpy arrays, in place
    (see sad_densify_prune): statistics over the per-pixel map, split, prune, seed
    the map, reset the removal accumulator.  sites, m, v float32 [10][stride];
    removal float32 [stride]; cand uint32 [H][W][8]; target float32 [H][W][3].
    Returns (new n_slots, status), status 0 or SAD_ERR_CAPACITY."""
    import numpy as np
    for name, a, dt in (("sites", sites, np.float32), ("m", m, np.float32), ("v", v, np.float32),
                        ("removal", removal, np.float32), ("cand", cand, np.uint32),
                        ("target", target, np.float32)):
        if not isinstance(a, np.ndarray) or a.dtype != dt or not a.flags["C_CONTIGUOUS"]:
            raise TypeError(f"{name} must be a C-contiguous numpy {np.dtype(dt).name} array")
    stride = sites.shape[1]
    if sites.shape[0] != NPARAM or m.shape != sites.shape or v.shape != sites.shape or \
            removal.shape != (stride,) or target.shape != (H, W, 3) or cand.shape != map_shape(W, H):
        raise ValueError("densify_prune: inconsistent shapes")
    ns = ctypes.c_int(n_slots)
    c = (cfg or BudgetConfig()).to_c()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rc = lib().sad_densify_prune(p(sites), p(m), p(v), p(removal), ctypes.byref(ns), capacity, stride, p(cand), W,
                                 H, p(target), ctypes.byref(c), ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF))
    if rc not in (SAD_OK, SAD_ERR_CAPACITY):
        raise SadError("sad_densify_prune", rc)
    return ns.value, rc


def densify_prune_stats(sites, m, v, n_slots, capacity, stats, removal, cand, W, H, target,
                        cfg: BudgetConfig | None = None, cell=1, want_seeds=False):
    """Host-side split/prune on numpy arrays with given statistics, in place (see
    sad_densify_prune_stats).

    sites, m, v: float32 [10][stride]; stats float32 [stride][8]; removal float32
    [stride]; cand uint32 [Hm][Wm][8] (map_shape) or None; target float32 [H][W][3].
    Returns (new n_slots, n_split, n_pruned, status) -- status is 0 or
    SAD_ERR_CAPACITY -- and, with want_seeds, the seeding (entry, ID) pairs as a
    uint32 [n][2] array, grouped by entry and in write order within an entry."""
    import numpy as np
    arrays = [("sites", sites, np.float32), ("m", m, np.float32), ("v", v, np.float32),
              ("stats", stats, np.float32), ("removal", removal, np.float32), ("target", target, np.float32)]
    if cand is not None:
        arrays.append(("cand", cand, np.uint32))
    for name, a, dt in arrays:
        if not isinstance(a, np.ndarray) or a.dtype != dt or not a.flags["C_CONTIGUOUS"]:
            raise TypeError(f"{name} must be a C-contiguous numpy {np.dtype(dt).name} array")
    stride = sites.shape[1]
    if m.shape != sites.shape or v.shape != sites.shape or stats.shape != (stride, STAT_LD) or \
            removal.shape != (stride,) or target.shape != (H, W, 3) or \
            (cand is not None and cand.shape != map_shape(W, H, cell)):
        raise ValueError("densify_prune: inconsistent shapes")
    ns = ctypes.c_int(n_slots)
    nsp = ctypes.c_int(0)
    npr = ctypes.c_int(0)
    c = (cfg or BudgetConfig()).to_c()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a is not None else None
    seeds = np.empty((5 * stride + 1, 2), dtype=np.uint32) if want_seeds else None
    nseed = ctypes.c_long(0)
    rc = lib().sad_densify_prune_stats(p(sites), p(m), p(v), stride, capacity, ctypes.byref(ns), p(stats),
                                       p(removal), p(cand), W, H, cell, p(target), ctypes.byref(c),
                                       ctypes.byref(nsp), ctypes.byref(npr), p(seeds),
                                       seeds.shape[0] if want_seeds else 0, ctypes.byref(nseed))
    if rc not in (SAD_OK, SAD_ERR_CAPACITY):
        raise SadError("sad_densify_prune_stats", rc)
    if want_seeds:
        return ns.value, nsp.value, npr.value, rc, seeds[:nseed.value]
    return ns.value, nsp.value, npr.value, rc


# ------------------------------------------------- evaluation format and queries
def new_eval(capacity: int, device="cuda"):
    """Storage for the evaluation format: words uint32 [capacity][4] (held as
    int32) and the per-image header float32 [4]."""
    return (torch.zeros((max(capacity, 1), 4), dtype=torch.int32, device=device),
            torch.zeros(4, dtype=torch.float32, device=device))


def _words(words, n_slots):
    if words.dim() != 2 or words.shape[1] != 4 or words.shape[0] < n_slots:
        raise ValueError("words must be int32 [>= n_slots][4]")
    return _dev(words, "words", _U32)


def _header(header):
    if header.numel() != 4:
        raise ValueError("header must hold 4 float32")
    return _dev(header, "header", _F32)


def eval_encode(sites, n_slots, W, H, words, header, stream=None):
    """Packs slots [0, n_slots) into the 16-byte evaluation format (see sad_eval_encode)."""
    sp, stride = _sites(sites, n_slots)
    _check("sad_eval_encode", lib().sad_eval_encode(sp, n_slots, stride, W, H, _words(words, n_slots),
                                                    _header(header), _stream(stream)))


def eval_decode(words, header, n_slots, W, H, sites, stream=None):
    """The site planes the evaluation words stand for (see sad_eval_decode)."""
    sp, stride = _sites(sites, n_slots)
    _check("sad_eval_decode", lib().sad_eval_decode(_words(words, n_slots), _header(header), n_slots, W, H, sp,
                                                    stride, _stream(stream)))


def eval_query(words, header, n_slots, cand, W, H, points, out_rgb, stream=None, cell=1):
    """Colour at arbitrary points (float32 [n][2], px) from the evaluation words and
    a candidate map (see sad_eval_query)."""
    if points.dim() != 2 or points.shape[1] != 2:
        raise ValueError("points must be float32 [n][2]")
    n = points.shape[0]
    c = _dev(cand, "cand", _U32, map_shape(W, H, cell))
    pp = _dev(points, "points", _F32)
    o = _dev(out_rgb, "out_rgb", _F32, (n, 3))
    _check("sad_eval_query", lib().sad_eval_query(_words(words, n_slots), _header(header), n_slots, c, W, H, cell,
                                                  pp, n, o, _stream(stream)))


def jump_schedule(W: int, H: int, n: int, cell: int = 1) -> list:
    """Jumps for n passes: B/2, B/4, ..., 1, then 1, with B = 2^ceil(log2 max(Wm,Hm))
    in map entries (paperlayer.ai summary, section 4 "Candidate maintenance"; B is
    our reading)."""
    Hm, Wm, _ = map_shape(W, H, cell)
    B = 1 << max(0, (max(Wm, Hm) - 1).bit_length())
    out, k = [], B // 2
    for _ in range(n):
        out.append(max(k, 1))
        k //= 2
    return out


def new_grad(stride: int, device="cuda") -> torch.Tensor:
    """Zeroed gradient records (cached form), float32 [stride][16]."""
    return torch.zeros((stride, GRAD_LD), dtype=torch.float32, device=device)


def new_grad_planes(stride: int, device="cuda") -> torch.Tensor:
    """Zeroed gradient planes (site-buffer form), float32 [11][stride]."""
    return torch.zeros((NACC, stride), dtype=torch.float32, device=device)


def apply_seeds(cand, W, H, seeds, stream=None, cell=1):
    """Applies seeding pairs (uint32 [n][2] as int32, grouped by entry) to a map on
    the GPU (see sad_apply_seeds)."""
    c = _dev(cand, "cand", _U32, map_shape(W, H, cell))
    if seeds.dim() != 2 or seeds.shape[1] != 2:
        raise ValueError("seeds must be int32 [n][2]")
    sd = _dev(seeds, "seeds", _U32)
    _check("sad_apply_seeds", lib().sad_apply_seeds(c, W, H, cell, sd, seeds.shape[0], _stream(stream)))


def grad_planes(grad: torch.Tensor):
    """The 11 accumulators as planes [11][stride] (a host-side view for inspection)."""
    return grad[:, :NACC].t()


def new_map(W: int, H: int, device="cuda", cell: int = 1) -> torch.Tensor:
    """An all-sentinel candidate map (uint32 [Hm][Wm][8] held as int32)."""
    return torch.full(map_shape(W, H, cell), -1, dtype=torch.int32, device=device)


class Fitter:
    """One SAD fitting state on the GPU and its iteration: propagate, render
    forward, render backward, Adam (which also refreshes the site records the
    image-space kernels read).  Everything runs in libsad kernels on one stream;
    nothing crosses to the host inside an iteration.

    The coarse-to-fine warm-up (jumps B/2 .. 1) runs before the first render
    (`warmup="first"`), or one pass per iteration (`"interleaved"`); after it the
    candidate field is refreshed every `refresh_every` iterations with
    `passes_per_refresh` propagation passes (paperlayer.ai summary, section 4 and
    B.3: the long-range warm-up comes first and the regular updates after it; both
    the update frequency and the passes per update are exposed, and 8-16
    iterations between updates left the final PSNR unchanged there).  Rendering
    and back-propagating through the half-built lists of an interleaved warm-up
    is what the first iterations spend most of their time on: a tile's lists then
    name a thousand random sites.  The pass counter drives the jump schedule and the
    injection's pass index.  `cell` > 1 keeps the candidate map on the downscaled
    grid of B.3 "Candidate field" (ceil(W/cell) x ceil(H/cell) lists).  With
    `packed` the candidate passes read the 16-byte float16 candidate-site buffer
    of B.2 "Packed candidate sites" (Adam refreshes it with the records).  With
    `screen` (the default) the candidate passes discard candidates that provably
    cannot enter a list before fetching their records (sad_site_screen; the same
    lists)."""

    def __init__(self, sites: torch.Tensor, n_slots: int, target: torch.Tensor, W: int, H: int,
                 n_inject: int = 4, seed: int = 4, adam: AdamConfig | None = None, cand: torch.Tensor | None = None,
                 refresh_every: int = 1, passes_per_refresh: int = 1, cell: int = 1, packed: bool = False,
                 screen: bool = True, warmup: str = "first"):
        if refresh_every < 1 or passes_per_refresh < 0:
            raise ValueError("refresh_every >= 1 and passes_per_refresh >= 0")
        if warmup not in ("first", "interleaved"):
            raise ValueError("warmup is 'first' or 'interleaved'")
        self.warmup = warmup
        dev = sites.device
        self.W, self.H, self.n_slots, self.n_inject, self.seed = W, H, n_slots, n_inject, seed
        self.cell = cell
        self.Hm, self.Wm, _ = map_shape(W, H, cell)
        self.refresh_every, self.passes_per_refresh = refresh_every, passes_per_refresh
        self.passes = 0
        self.warm_end = 0  # first iteration after the warm-up passes
        self.sites = sites
        self.target = target
        stride = sites.shape[1]
        self.m = torch.zeros((NPARAM, stride), dtype=torch.float32, device=dev)
        self.v = torch.zeros((NPARAM, stride), dtype=torch.float32, device=dev)
        self.grad = torch.zeros((stride, GRAD_LD), dtype=torch.float32, device=dev)
        self.rec = new_records(stride, dev)
        site_records(sites, n_slots, self.rec)
        self.packed = None
        if packed:
            self.packed = new_packed(stride, dev)
            pack_sites(sites, n_slots, self.packed)
        self.scr = None
        if screen:
            self.scr = new_screen(stride, dev)
            site_screen(sites, n_slots, W, H, self.scr)
        self.maps = [cand if cand is not None else new_map(W, H, dev, cell), new_map(W, H, dev, cell)]
        self.cur = 0
        self.rgb = torch.empty((H, W, 3), dtype=torch.float32, device=dev)
        self.loss = new_loss(dev)
        self.adam = (adam or AdamConfig()).to_c(W, H)
        self.it = 0
        self.sched_cache: dict = {}

    @property
    def cand(self) -> torch.Tensor:
        return self.maps[self.cur]

    def jump_at(self, it: int) -> int:
        B = 1 << max(0, (max(self.Wm, self.Hm) - 1).bit_length())
        return max(1, (B // 2) >> it) if it < 64 else 1

    @property
    def sel(self) -> torch.Tensor:
        """The site buffer the candidate passes read."""
        return self.packed if self.packed is not None else self.rec

    def refresh_records(self, stream=None):
        """Recompute the site records (and the packed buffer) after changing
        `sites` outside Adam."""
        site_records(self.sites, self.n_slots, self.rec, stream)
        if self.packed is not None:
            pack_sites(self.sites, self.n_slots, self.packed, stream)
        if self.scr is not None:
            site_screen(self.sites, self.n_slots, self.W, self.H, self.scr, stream)

    def propagate(self, jump: int, pass_index: int, stream=None):
        topk_propagate_rec(self.sel, self.n_slots, self.maps[self.cur], self.maps[1 - self.cur], self.W, self.H,
                           jump, pass_index, self.seed, self.n_inject, stream, self.cell, self.scr)
        self.cur = 1 - self.cur

    def step(self, stream=None):
        """One iteration (the hot path): propagate, render forward and backward
        (one fused launch that writes the image and the gradients), Adam."""
        it = self.it
        warm = (max(self.Wm, self.Hm) - 1).bit_length()  # log2 B passes with jumps B/2 .. 1
        if self.passes < warm:
            # the coarse-to-fine warm-up: all of it before the first render, or
            # one pass per iteration
            while self.passes < warm:
                self.propagate(self.jump_at(self.passes), self.passes, stream)
                self.passes += 1
                if self.warmup == "interleaved":
                    break
            self.warm_end = it + 1
        elif (it - self.warm_end) % self.refresh_every == 0:
            for _ in range(self.passes_per_refresh):
                self.propagate(self.jump_at(self.passes), self.passes, stream)
                self.passes += 1
        render_bwd_rec(self.rec, self.n_slots, self.cand, self.target, self.W, self.H, self.grad, self.loss,
                       self.rgb, stream, self.cell)
        adam_step_rec(self.sites, self.m, self.v, self.grad, self.n_slots, it + 1, self.W * self.H, self.W, self.H,
                      self.adam, self.rec, stream, self.packed, self.scr)
        self.it += 1

    def densify(self, cfg: BudgetConfig | None = None, stream=None):
        """Budget control between iterations: per-site statistics on the GPU
        (sad_densify_stats), split/prune on the host (sad_densify_prune) using the
        removal deltas accumulated since the last call, then the site records are
        rebuilt and the removal accumulators cleared.  Returns (n_split, n_pruned).

        Only what the host routine reads or changes crosses PCIe, through pinned
        buffers kept between calls: sites, moments, statistics and removal deltas
        (the target once, and again only if the tensor is modified).  The map
        stays on the GPU: the routine reports the entries it seeds with the new
        sites, and sad_apply_seeds writes them there (a list keeps distinct IDs)."""
        import numpy as np
        dev = self.sites.device
        stride = self.sites.shape[1]
        stats = torch.zeros((stride, STAT_LD), dtype=torch.float32, device=dev)
        densify_stats(self.rec, self.n_slots, self.cand, self.target, self.W, self.H, stats, stream, self.cell)
        if getattr(self, "_host", None) is None:
            pin = lambda t: torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            self._host = {"sites": pin(self.sites), "m": pin(self.m), "v": pin(self.v), "stats": pin(stats),
                          "removal": torch.empty(stride, dtype=torch.float32, pin_memory=True),
                          "target": pin(self.target)}
        h = self._host
        copies = [("sites", self.sites), ("m", self.m), ("v", self.v), ("stats", stats),
                  ("removal", self.grad[:, NACC - 1])]
        tkey = (self.target.data_ptr(), self.target._version)
        if getattr(self, "_host_target", None) != tkey:  # the target crosses once, not per call
            copies.append(("target", self.target))
            self._host_target = tkey
        for k, src in copies:
            h[k].copy_(src, non_blocking=True)
        torch.cuda.synchronize(dev)
        hn = {k: t.numpy() for k, t in h.items()}
        n, n_split, n_pruned, _, seeds = densify_prune_stats(hn["sites"], hn["m"], hn["v"], self.n_slots, stride,
                                                             hn["stats"], hn["removal"], None, self.W, self.H,
                                                             hn["target"], cfg, self.cell, want_seeds=True)
        for k, dst in (("sites", self.sites), ("m", self.m), ("v", self.v)):
            dst.copy_(h[k], non_blocking=True)
        if len(seeds):
            apply_seeds(self.cand, self.W, self.H, torch.from_numpy(seeds.view(np.int32)).to(dev), stream,
                        self.cell)
        self.grad[:, NACC - 1].zero_()
        self.n_slots = n
        self.refresh_records(stream)
        torch.cuda.synchronize(dev)  # the pinned buffers are reused by the next call
        return n_split, n_pruned
