"""Oracle of the 16-byte packed evaluation format -- TEST INFRASTRUCTURE ONLY (only
the tests, the package smoke check and the benchmark's CPU baseline use it).

Pages: paperlayer.ai summary, Appendix B.2 "Packed storage for evaluation" (all
ten values in four 32-bit words, quantised position, colour, temperature, radius
and direction; per-image min/scale for log tau and r); 69574.cn article, section 5
(15-bit fixed-point coordinates, colour in 11/11/10 bits, 16 bits each for the
temperature and the radius, a 16-bit direction angle, the anisotropy in float16).

Readings (the pages give the field widths, nothing more):
  E1 words: w0 = qx | qy << 15 | inactive << 31 (bit 30 zero); w1 = qR | qG << 11
     | qB << 22; w2 = q_logtau | q_r << 16; w3 = q_angle | f16(a) << 16.  An
     inactive slot (x < 0) is w0 = 1 << 31, w1 = w2 = w3 = 0.
  E2 quantisation in float32: t = v * scale (one rounded product; for log tau and r
     t = (v - min) * inv, two rounded operations), q = rint(t) (nearest even),
     then q < 0 or NaN -> 0 and q > qmax -> qmax.
       x: scale = 32767 / W, y: 32767 / H (qmax 32767);
       R, G: scale 2047, B: 1023 (qmax the same);
       log tau, r: min and max over the active slots' finite values, inv =
       65535 / (max - min) (0 when max <= min), qmax 65535.
  E3 direction: the metric depends on the axis only (u and -u give the same G),
     so the angle theta = atan2(dy, dx) folded into [0, pi) is stored:
     t = theta * 65536 / pi in float64 (float32 atan2 implementations differ by
     an ulp, which would flip the code near ties), q = rint(t) mod 65536; a
     degenerate direction (dx^2 + dy^2 < 1e-30) stores 0.
  E4 a: IEEE binary16, nearest even.
  E5 header (per image): float32 [lt_min, lt_step, r_min, r_step] with step =
     (max - min) / 65535 (a zero extreme is stored as +0).
  E6 decoding in float32, each operation rounded separately: x = qx * (W / 32767),
     y = qy * (H / 32767), R = qR * (1 / 2047), G likewise, B = qB * (1 / 1023),
     log tau = lt_min + q * lt_step, r = r_min + q * r_step, theta = q * (pi / 65536),
     dir = (cos theta, sin theta) (float64 here), a from binary16; an inactive slot
     decodes to x = y = -1.
"""
import numpy as np

X, Y, LOGTAU, R, CR, CG, CB, DX, DY, A = range(10)
f32 = np.float32
QPOS, QRG, QB, Q16, QANG = 32767, 2047, 1023, 65535, 65536
ANG_STEP = f32(np.pi / 65536)  # float64 quotient rounded once to float32


def _quant(t, qmax):
    t = np.rint(np.asarray(t, dtype=np.float32))
    t = np.where(~(t >= 0), f32(0), t)
    return np.minimum(t, f32(qmax)).astype(np.uint32)


def _range(v, active):
    v = v[active & np.isfinite(v)]
    if v.size == 0:
        return f32(0), f32(0)
    return f32(v.min()) + f32(0), f32(v.max()) + f32(0)  # a zero extreme is +0


def eval_encode(sites, n_slots, W, H):
    """Returns (words uint32 [n_slots][4], header float32 [4])."""
    S = np.asarray(sites, dtype=np.float32)[:, :n_slots]
    active = ~(S[X] < 0)
    lt_m, lt_M = _range(S[LOGTAU], active)
    r_m, r_M = _range(S[R], active)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        lt_inv = f32(Q16) / f32(lt_M - lt_m) if lt_M > lt_m else f32(0)
        r_inv = f32(Q16) / f32(r_M - r_m) if r_M > r_m else f32(0)
        header = np.array([lt_m, f32(lt_M - lt_m) / f32(Q16), r_m, f32(r_M - r_m) / f32(Q16)], dtype=np.float32)
        qx = _quant(S[X] * (f32(QPOS) / f32(W)), QPOS)
        qy = _quant(S[Y] * (f32(QPOS) / f32(H)), QPOS)
        qr_ = _quant(S[CR] * f32(QRG), QRG)
        qg = _quant(S[CG] * f32(QRG), QRG)
        qb = _quant(S[CB] * f32(QB), QB)
        qlt = _quant((S[LOGTAU] - lt_m) * lt_inv, Q16)
        qrad = _quant((S[R] - r_m) * r_inv, Q16)
        dx, dy = S[DX].astype(np.float64), S[DY].astype(np.float64)
        th = np.arctan2(dy, dx)
        th = np.where(th < 0, th + np.pi, th)
        t = np.rint(th * (QANG / np.pi))
        t = np.where(np.isfinite(t), t, 0.0)
        qa = (t.astype(np.int64) % QANG).astype(np.uint32)
        qa = np.where(dx * dx + dy * dy < 1e-30, np.uint32(0), qa)
        ha = S[A].astype(np.float16).view(np.uint16).astype(np.uint32)
    w = np.empty((n_slots, 4), dtype=np.uint32)
    w[:, 0] = qx | (qy << 15)
    w[:, 1] = qr_ | (qg << 11) | (qb << 22)
    w[:, 2] = qlt | (qrad << 16)
    w[:, 3] = qa | (ha << 16)
    w[~active] = 0
    w[~active, 0] = np.uint32(1 << 31)
    return w, header


def eval_decode(words, header, n_slots, W, H, stride=None):
    """The float sites the evaluation format stands for, [10][stride] float64 (the
    values of E6: float32 arithmetic except cos/sin), inactive slots x = y = -1."""
    w = np.asarray(words, dtype=np.uint32)[:n_slots]
    hd = np.asarray(header, dtype=np.float32)
    S = np.zeros((10, stride or n_slots), dtype=np.float64)
    S[X] = S[Y] = -1.0
    qx = (w[:, 0] & 0x7FFF).astype(np.float32)
    qy = ((w[:, 0] >> 15) & 0x7FFF).astype(np.float32)
    x = qx * (f32(W) / f32(QPOS))
    y = qy * (f32(H) / f32(QPOS))
    cr = (w[:, 1] & 0x7FF).astype(np.float32) * (f32(1) / f32(QRG))
    cg = ((w[:, 1] >> 11) & 0x7FF).astype(np.float32) * (f32(1) / f32(QRG))
    cb = (w[:, 1] >> 22).astype(np.float32) * (f32(1) / f32(QB))
    lt = hd[0] + (w[:, 2] & 0xFFFF).astype(np.float32) * hd[1]
    rad = hd[2] + (w[:, 2] >> 16).astype(np.float32) * hd[3]
    th = (w[:, 3] & 0xFFFF).astype(np.float32) * ANG_STEP
    a = (w[:, 3] >> 16).astype(np.uint16).view(np.float16).astype(np.float32)
    act = (w[:, 0] >> 31) == 0
    for f, v in ((X, x), (Y, y), (LOGTAU, lt), (R, rad), (CR, cr), (CG, cg), (CB, cb), (A, a)):
        S[f, :n_slots] = np.where(act, v.astype(np.float64), S[f, :n_slots])
    S[DX, :n_slots] = np.where(act, np.cos(th.astype(np.float64)), 0.0)
    S[DY, :n_slots] = np.where(act, np.sin(th.astype(np.float64)), 0.0)
    return S
