/*
 * sad.h -- C ABI of libsad, the MI355X (gfx950) hot path of Soft Anisotropic
 * Diagrams (SAD): top-K candidate maintenance (propagation with injection, the
 * optional jump-flood prepass, the exact top-K; per pixel or on a downscaled
 * grid), the temperature-softmax render, its analytic backward, Adam, budget
 * control, the packed candidate-site buffer, and the 16-byte evaluation format
 * with random-access point queries.
 *
 * Sources (the pages the method is described on):
 *   [SUM]   paperlayer.ai summary of arXiv:2604.21984v2, sections 3-5 and Appendix B
 *   [NOTE]  woaixuexisr.github.io reading note, "Key designs" 1-4
 *   [PROJ]  luckyiyi.github.io/SAD project page, "Method"
 *   [PRESS] 69574.cn article, sections 3-5
 *
 * Two forms of the iteration's calls
 * ----------------------------------
 * The site-buffer form -- sad_topk_propagate, sad_render_fwd, sad_render_bwd,
 *   sad_adam_step, sad_densify_prune -- takes the site buffer itself (`sites`,
 *   ten planes), gradients as eleven planes and a scalar loss: the buffers
 *   [SUM] B.2 and B.4 describe, nothing derived.  Only site I/O has to cross to
 *   the host ([SUM] B.8).
 * The cached form -- the same names with the suffix _rec (and
 *   sad_densify_prune_stats) -- reads derived per-site caches (`rec`, `packed`)
 *   that Adam keeps current, writes the gradients as one 64-byte record per site,
 *   and takes a `cell` for the downscaled candidate grid.  It computes the same
 *   quantities (the scores, lists and images bit for bit when the cache is
 *   current) with fewer scattered accesses; the fit driver and the benchmark use
 *   it.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership.  The caller owns every buffer.  The library allocates no device
 *   memory (the host budget-control routines use temporary host memory and host
 *   threads) and keeps no state between calls, so calls are reentrant.
 * Pointers.  Arguments named `sites`, `rec`, `packed`, `cand*`, `out_rgb`,
 *   `target`, `grad`, `m`, `v`, `loss_sum`, `stats`, `scr`, `seeds`, `entries`,
 *   `out`, `words`, `header` and `points` are DEVICE pointers (HBM of the current HIP
 *   device), except in sad_densify_prune and sad_densify_prune_stats, which work
 *   on HOST arrays.  `cfg` is a HOST pointer, read before the call returns.
 * Streams.  Device work is enqueued asynchronously on `stream` (a hipStream_t
 *   passed as void*; NULL = the legacy default stream).  A return of SAD_OK means
 *   the launch was accepted, not that the kernel finished.
 * Errors.  Every call returns SAD_OK (0) or a negative sad_status.  Arguments
 *   are checked on the host before anything is launched; on an argument error
 *   nothing is launched and no buffer is touched.  A launch failure reported by
 *   the HIP runtime returns SAD_ERR_DEVICE.  No C++ exception crosses the ABI.
 *
 * Layouts
 * -------
 * sites : float [SAD_NPARAM][stride] -- ten planes ("structure of arrays"), the
 *         ten float32 values per site of [SUM] B.2, in the field order of
 *         [PRESS] 5: x, y, log_tau, r, R, G, B, dir_x, dir_y, a.  Positions and r
 *         are in pixels; tau = exp(log_tau).  Slots [0, n_slots) are in use; a slot
 *         whose x < 0 is inactive and every kernel ignores it ([SUM] B.2, B.5).
 *         4-byte aligned.
 * cand  : uint32 [Hm][Wm][SAD_K] -- the candidate map: site IDs per map entry
 *         ([SUM] B.2 keeps K = 8 IDs per entry in two 4-channel textures; here one
 *         32-byte record per entry), SAD_INVALID marks an empty entry.  16-byte
 *         aligned.  Lists written by this library hold distinct IDs in ascending
 *         (d, ID) order.
 *         Grid ([SUM] B.3 "Candidate field", cached form only): the entries that
 *         take `cell` = c cover c x c pixels, Wm = ceil(W/c), Hm = ceil(H/c);
 *         pixel (col, row) is rendered with the list of entry (col/c, row/c)
 *         (integer division), and an entry's list is selected at its centred UV,
 *         ((cx + 1/2) W/Wm, (cy + 1/2) H/Hm) px (float32: W/Wm and H/Hm rounded
 *         once, then one add and one multiply).  c = 1 is the per-pixel map,
 *         [H][W][8], evaluated at pixel centres -- the map of the site-buffer
 *         form.  1 <= c <= 65535; every call that reads or writes the map takes
 *         the same c.
 * images: float [H][W][3] (RGB, linear).
 * grad  : site-buffer form: float [SAD_NACC][stride] -- eleven planes: the ten
 *         gradients in site order, then the removal delta ([SUM] B.4: 11
 *         accumulators per site).  4-byte aligned.
 *         Cached form: float [stride][SAD_GRAD_LD] -- one 64-byte record per site:
 *         the ten gradients at [0,10), the removal delta at [10], words [11,16)
 *         unused and never written; 16-byte aligned.  (The atomics that flush one
 *         site's 11 sums then share one cache line.)
 * m, v  : float [SAD_NPARAM][stride] Adam moments.
 * rec   : float [n_slots][SAD_REC_LD] -- one 64-byte record per site, derived from
 *         `sites` (sad_site_records) and refreshed by sad_adam_step_rec; a random
 *         access to a site then costs a few contiguous loads:
 *           [0..4)   x, y, r, Ux        [4..8)   Uy, Vx, Vy, tau
 *           [8..12)  R, G, B, 1/|dir|   [12..16) ux, uy, E, 1/E
 *         with u = dir/|dir| (u = (1,0) if |dir|^2 < 1e-30; 1/|dir| is then 0),
 *         E = e^a, tau = e^{log tau}, U = e^{a/2} u, V = e^{-a/2} u, so that
 *         ||delta||_G^2 = (U.delta)^2 + (Vx delta_y - Vy delta_x)^2.  The first
 *         32 bytes are the fp32 counterpart of the compact per-site buffer the
 *         pages' candidate-update kernels read ([SUM] B.2 "Packed candidate
 *         sites").  A slot with x < 0 stays inactive.  16-byte aligned.  It is a
 *         cache the caller keeps in step with `sites`: recompute it after any
 *         change made outside sad_adam_step_rec.  Stale records give results for
 *         the sites they were made from.
 * scr   : uint32 [n_slots] -- the candidate screen, one 4-byte word per site that
 *         bounds where the site can score (cached form only).  Its cells divide
 *         the image into 4096 x 4096: bits 0..11 qx = floor(x 4096/W), bits 12..23
 *         qy = floor(y 4096/H) (the site lies in that cell), bits 24..27 ca with
 *         2^(ca/2) >= e^{|a|/2}, bits 28..31 cr with 2^(cr-8) >= 2^(ca/2) max(r,0)
 *         (cr = 0: 0); ca = 15 or cr = 15: no bound.  Since ||x - p||_G >=
 *         ||x - p|| / e^{|a|/2}, a selection pass can discard a candidate that
 *         provably scores after its list's K-th entry without fetching its
 *         record (propagation screens the injected IDs, uniform over the image,
 *         and the IDs its site table could not hold); the lists are the same bits
 *         with or without the screen.  It
 *         bounds float32 scores of the sites, so it serves selection from the
 *         records; with the packed buffer (float16-rounded sites) it is ignored.  A
 *         cache like `rec`: sad_site_screen writes it, sad_adam_step_rec refreshes
 *         it.  4-byte aligned.
 * packed: uint32 [n_slots][SAD_PACK_LD] -- the packed candidate-site buffer
 *         ([SUM] B.2 "Packed candidate sites": 16 bytes per site of float16 pairs,
 *         read by the candidate-update kernels to save bandwidth): word 0 = (x, y),
 *         word 1 = (log tau, r), word 2 = (dir_x, dir_y), word 3 = (a, 0), the
 *         first value of each pair in the low 16 bits; IEEE binary16, rounded to
 *         nearest even, overflow to infinity; an inactive slot (x < 0) packs
 *         x = -1.  16-byte aligned.  Selection entry points given it (sel_fmt =
 *         SAD_SEL_PACKED16) rank the sites as if their seven packed fields were
 *         rounded to binary16: the same score, ranking and filters, evaluated in
 *         float32 from the decoded values.  A cache like `rec`: sad_pack_sites
 *         writes it, sad_adam_step_rec refreshes it.
 * Pixel (col,row) is rendered at (col+0.5, row+0.5) px ([SUM] B.3 evaluates at
 * centred cells).  Limits: 1 <= W, H <= 65535 (W or H = 0 is an empty image: a
 * no-op returning SAD_OK after the scalar arguments are checked; its pointers
 * may then be NULL); 0 <= n_slots <= stride.
 *
 * Score ([NOTE] design 1, [PROJ] "Method"):
 *   d(x,i) = s * ||x - p_i||_{G_i} - s * r_i,  s = 1 / max(H, W),
 *   G_i = e^{a_i} u u^T + e^{-a_i} v v^T,  u = dir/|dir| (u = (1,0) if |dir|^2 < 1e-30),
 *   v = (-u_y, u_x), so det G_i = 1 ([SUM] section 4).
 * Candidates are ranked by (d ascending, site ID ascending).
 */
#ifndef SAD_H
#define SAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAD_ABI_VERSION 7
#define SAD_K 8
#define SAD_INVALID 0xffffffffu
#define SAD_NPARAM 10
#define SAD_NACC 11
#define SAD_GRAD_LD 16
#define SAD_REC_LD 16
#define SAD_STAT_LD 8
#define SAD_MAX_INJECT 16
#define SAD_MAX_DIM 65535
#define SAD_LOSS_SLOTS 64 /* partial sums of the loss output of sad_render_bwd_rec */
#define SAD_PACK_LD 4     /* uint32 words per site of the packed candidate-site buffer */

/* Site formats the cached selection entry points read (`sel_fmt`). */
#define SAD_SEL_REC64 0    /* `rec`: the 64-byte site records                          */
#define SAD_SEL_PACKED16 1 /* `rec`: the 16-byte packed candidate-site buffer (packed) */

enum sad_status {
    SAD_OK = 0,
    SAD_ERR_ARG = -1,           /* a size, count or pointer argument is invalid        */
    SAD_ERR_ALIGN = -2,         /* a pointer is not aligned as its layout requires     */
    SAD_ERR_DEVICE = -3,        /* the HIP runtime rejected a launch                    */
    SAD_ERR_CAPACITY = -4,      /* a result would not fit the given capacity           */
    SAD_ERR_UNIMPLEMENTED = -5  /* reserved                                             */
};

enum sad_param { SAD_X, SAD_Y, SAD_LOGTAU, SAD_R, SAD_CR, SAD_CG, SAD_CB, SAD_DIRX, SAD_DIRY, SAD_A };

/* Adam hyper-parameters: one learning rate per site parameter, in site order,
 * and the box the positions are clamped to after each step, [0, x_max] x
 * [0, y_max] (the image size in pixels: a site leaving it would cross into the
 * x < 0 "inactive" marker of [SUM] B.2); 0 < x_max, y_max <= SAD_MAX_DIM. */
typedef struct sad_adam_cfg {
    float lr[SAD_NPARAM];
    float beta1, beta2, eps;
    float x_max, y_max;
} sad_adam_cfg;

/* Budget control ([SUM] B.5; [NOTE] design 4).  The pages do not reproduce their
 * constants (Tables B11/B12 are referenced, not given); the defaults in the
 * Python binding are ours. */
typedef struct sad_budget_cfg {
    float split_frac; /* fraction of the active sites split per call                  */
    float prune_frac; /* fraction of the active sites pruned per call                 */
    float alpha;      /* split score E / max(m, min_mass)^alpha                       */
    float min_mass;   /* mass (in pixels) below which a site's covariance is not used */
    float shrink;     /* children: r *= shrink, log tau += log(shrink)                */
} sad_budget_cfg;

/* SAD_ABI_VERSION of the loaded library. */
int sad_abi_version(void);

/* Static text for a status code (never NULL). */
const char *sad_status_string(int status);

/* ======================================================================== */
/* The iteration on the site buffer                                         */
/* ======================================================================== */

/*
 * sad_topk_propagate -- one propagation pass of the per-pixel candidate map.
 * [NOTE] design 3: C~_t(x) = C_{t-1}(x) U P_t(x) U G_t(x), keep the top-K under d;
 * [SUM] section 4: self plus 4 neighbours at the current jump, plus a small
 * random set of global IDs; [SUM] B.3 packs the pass index (low 16 bits) and the
 * jump (high 16 bits) into one word that, with the pixel ID, seeds xorshift.
 *
 * For every pixel x the candidates are: its own list in cand_in, the lists of
 * the pixels x +- (jump, 0) and x +- (0, jump) that lie inside the image, and
 * `n_inject` IDs drawn as follows (identical on every implementation):
 *   pw = (jump << 16) | (pass_index & 0xffff);  pix = row*W + col;
 *   h  = pcg(pcg(pcg(seed) ^ pw) ^ pix)   (pcg: Jarzynski & Olano, JCGT 2020)
 *   x  = h ? h : 0x9e3779b9;  repeat n_inject times: x = xorshift32(x) (13,17,5);
 *   id = (uint32)(((uint64)x * n_slots) >> 32).
 * Sentinels, IDs >= n_slots, inactive sites, non-finite scores and duplicates are
 * dropped; the K smallest by (d, ID) are written to cand_out in ascending order,
 * padded with SAD_INVALID.  The pass reads cand_in and writes cand_out (Jacobi).
 * The host chooses the schedule: jumps B/2, B/4, ..., 1 then 1 ([SUM] section 4).
 *   sites     device [10][stride], read-only
 *   cand_in   device [H][W][8] uint32, read-only, 16-byte aligned
 *   cand_out  device [H][W][8] uint32, written; must not overlap cand_in
 *   jump      1..65535;  n_inject 0..SAD_MAX_INJECT
 * Errors: SAD_ERR_ARG (bad sizes, jump, n_inject, NULL, overlapping maps),
 *         SAD_ERR_ALIGN (a map not 16-byte aligned), SAD_ERR_DEVICE.
 */
int sad_topk_propagate(const float *sites, int n_slots, int stride, const uint32_t *cand_in, uint32_t *cand_out, int W,
                       int H, int jump, uint32_t pass_index, uint32_t seed, int n_inject, void *stream);

/*
 * sad_render_fwd -- the temperature-softmax blend of each pixel's list, scored at
 * the pixel's centre.  [NOTE] design 2, [PROJ] "Method": l_i = -tau_i d_i,
 * w = softmax over the list, c(x) = sum_i w_i c_i; max-subtracted, invalid IDs
 * skipped, entries with a non-finite logit or colour skipped ([SUM] B.4).  A pixel
 * with no usable entry renders (0,0,0).  Duplicate IDs in a list each count.
 *   sites device [10][stride]; cand device [H][W][8] (16-byte aligned);
 *   out_rgb device [H][W][3] float, written.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_render_fwd(const float *sites, int n_slots, int stride, const uint32_t *cand, int W, int H, float *out_rgb,
                   void *stream);

/*
 * sad_render_bwd -- hand-derived gradients of L = sum_x ||c(x) - t(x)||^2 with
 * the map held fixed ([SUM] section 5 and B.4; [NOTE] design 4), accumulated
 * (+=) into the planes of `grad`.  Per pixel, g = 2(c - t); per usable entry k:
 *   dc_k = w_k g;  gamma_k = w_k g.(c_k - c);  dlog_tau_k = gamma_k l_k;
 *   dd_k = -tau_k gamma_k;  then through d = s q - s r to p, r, dir, a
 *   (through the normalisation u = dir/|dir|; zero for p, a, dir where q = 0).
 * Plane 10 receives the removal delta ||c_{-k} - t||^2 - ||c - t||^2, c_{-k} the
 * blend of the other entries renormalised (0 if none carries weight)
 * ([SUM] B.4-B.5).  Non-finite contributions are dropped.  Contributions are
 * summed per 16x16 tile in an LDS hash table keyed by site ID and flushed with
 * one atomic per site and accumulator per tile; an entry that finds no slot goes
 * straight to global atomics ([SUM] section 5, B.4).  Float atomics make the
 * summation order, hence the last bits, vary from run to run.
 *   sites device [10][stride]; cand device [H][W][8] (16-byte aligned);
 *   target device [H][W][3]; grad device [11][stride] float, +=;
 *   loss_sum device float[1] or NULL: += sum_x ||c(x) - t(x)||^2.
 * The caller zeroes `grad` once; sad_adam_step re-zeroes planes 0..9 each step;
 * plane 10 keeps accumulating until the caller (or sad_densify_prune) resets it.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN (cand not 16-byte aligned), SAD_ERR_DEVICE.
 */
int sad_render_bwd(const float *sites, int n_slots, int stride, const uint32_t *cand, const float *target, int W,
                   int H, float *grad, float *loss_sum, void *stream);

/*
 * sad_adam_step -- Adam (Kingma & Ba 2015) on the ten site parameters, with the
 * accumulated gradients divided by the pixel count ([SUM] B.4).  For each slot
 * i < n_slots with x >= 0 and each parameter j:
 *   g = grad[j][i] / n_pixels (non-finite -> 0);  m = b1 m + (1-b1) g;
 *   v = b2 v + (1-b2) g^2;  p -= lr_j (m / (1-b1^step)) / (sqrt(v / (1-b2^step)) + eps);
 * then x is clamped to [0, x_max] and y to [0, y_max] (cfg).  Planes 0..9 of grad
 * are zeroed for every slot < n_slots; plane 10 is left alone.  Inactive slots
 * keep p, m, v.
 *   sites, m, v device [10][stride] float (in/out); grad device [11][stride];
 *   step >= 1 (global, 1-based); n_pixels >= 1; cfg HOST pointer.
 * Errors: SAD_ERR_ARG, SAD_ERR_DEVICE.
 */
int sad_adam_step(float *sites, float *m, float *v, float *grad, int n_slots, int stride, int step, int n_pixels,
                  const sad_adam_cfg *cfg, void *stream);

/*
 * Budget-control rules shared by sad_densify_prune and sad_densify_prune_stats
 * ([SUM] B.5; [NOTE] design 4; [PRESS] 4).  Active sites: i < *n_slots with
 * x >= 0; A = their count.  Per-site statistics over the pixels x whose list holds
 * site i, with w its softmax weight at x, e(x) = ||c(x) - t(x)||^2 and
 * delta = x - p_i (float [stride][SAD_STAT_LD]):
 *   [0] sum w   [1] sum w e   [2] sum w e dx   [3] sum w e dy
 *   [4] sum w e dx^2   [5] sum w e dx dy   [6] sum w e dy^2   [7] unused
 *  (Counts below are computed in double from the float fields of cfg.)
 *  1. Split set: the floor(split_frac*A) active sites with the largest score
 *     S = stats[1] / max(stats[0], min_mass)^alpha (S > 0; ties -> lower ID).
 *  2. Prune set: the floor(prune_frac*A) active sites outside the split set with
 *     the smallest removal delta (ties -> lower ID; non-finite never pruned).
 *  3. Pruned sites get x = y = -1 (every kernel then ignores them, [SUM] B.5) and
 *     m = v = 0.
 *  4. Each split parent becomes two children offset by -o and +o from its
 *     position (clamped into [0,W]x[0,H]), along the principal axis of its
 *     error-weighted covariance, o = sqrt(lambda_max)/2 * e_max (e_max oriented
 *     with x > 0, or +y when vertical; equal eigenvalues give (1,0)).  When the mass
 *     is below min_mass or the covariance is degenerate, the axis is the Sobel
 *     gradient of the target's luminance at the parent's pixel ((1,0) if zero) and
 *     |o| = sqrt(max(mass, 1)/pi)/2 ([SUM] B.5: a local Sobel-type gradient).
 *     Children: colour = the target at their pixel, r *= shrink,
 *     log tau += log(shrink), other fields copied, m = v = 0 ([SUM] B.5).  Child A
 *     keeps the parent's slot; child B takes the lowest inactive slot below
 *     *n_slots, else slot *n_slots (then *n_slots grows) while below capacity.
 *  5. Seeding: child B's ID goes into the last place of the list of the map entry
 *     that contains it and of its 4 neighbour entries, so the next propagation
 *     pass ranks it -- unless that list already holds the ID (lists keep
 *     distinct IDs).  The entries are edited in split order.
 * The work runs on up to 8 host threads that the call starts and joins (one
 * thread if none can be started); the edits are those of one thread.
 */

/*
 * sad_densify_prune -- budget control on the HOST, from the site buffer: the
 * statistics above are computed here (float64, over every pixel of the
 * per-pixel map `cand`), then rules 1-5 are applied in place and the removal
 * accumulator of slots [0, *n_slots) (the new count) is reset to 0.
 *   sites, m, v HOST float [10][stride] (in/out); removal HOST float [stride]
 *   (in, reset; e.g. plane 10 of the gradient planes copied to the host);
 *   *n_slots in/out; capacity <= stride; cand HOST uint32 [H][W][8] (in/out:
 *   seeded); target HOST float [H][W][3]; cfg HOST.  `seed` is reserved: the
 *   rules take no random decision, so it does not change the result.
 * Errors: SAD_ERR_ARG (checked before anything is modified); SAD_ERR_CAPACITY when
 *  some selected sites could not be split for want of a free slot (everything
 *  that fitted is done).
 */
int sad_densify_prune(float *sites, float *m, float *v, float *removal, int *n_slots, int capacity, int stride,
                      uint32_t *cand, int W, int H, const float *target, const sad_budget_cfg *cfg, uint64_t seed);

/* ======================================================================== */
/* The iteration on derived site caches                                     */
/* ======================================================================== */

/*
 * sad_site_records -- writes the records (see `rec` above) of slots [0, n_slots)
 * from the site planes.
 *   sites device [10][stride] read-only; rec device [n_slots][16] float, written.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN (rec not 16-byte aligned), SAD_ERR_DEVICE.
 */
int sad_site_records(const float *sites, int n_slots, int stride, float *rec, void *stream);

/*
 * sad_pack_sites -- writes the packed candidate-site words (see `packed` above) of
 * slots [0, n_slots) from the site planes ([SUM] B.2: regenerated after
 * densification).
 *   sites device [10][stride] read-only; packed device [n_slots][4] uint32, written.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN (packed not 16-byte aligned), SAD_ERR_DEVICE.
 */
int sad_pack_sites(const float *sites, int n_slots, int stride, uint32_t *packed, void *stream);

/*
 * sad_site_screen -- writes the candidate screen (see `scr` above) of slots
 * [0, n_slots) of a W x H image from the site planes.
 *   sites device [10][stride] read-only; scr device uint32 [n_slots], written.
 *   W, H >= 1.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN (scr not 4-byte aligned), SAD_ERR_DEVICE.
 */
int sad_site_screen(const float *sites, int n_slots, int stride, int W, int H, uint32_t *scr, void *stream);

/*
 * sad_topk_propagate_rec -- sad_topk_propagate on a map of any cell size, reading
 * the site records (sel_fmt = SAD_SEL_REC64: the same lists as sad_topk_propagate
 * when the records are current) or the packed buffer (SAD_SEL_PACKED16), with the
 * candidate screen if `scr` is not NULL (the same lists, fewer record fetches).
 * For a grid map, x, jump and the neighbours are in map entries, pix = row*Wm +
 * col, and scores are taken at the entry's centred UV.
 *   rec       device, read-only: [n_slots][16] float or [n_slots][4] uint32
 *   scr       device uint32 [n_slots] or NULL, current for this W x H
 *   cand_in, cand_out device [Hm][Wm][8]; the rest as sad_topk_propagate.
 * Errors: SAD_ERR_ARG (also a bad cell or sel_fmt), SAD_ERR_ALIGN (a pointer not
 *         16-byte aligned, scr not 4-byte aligned), SAD_ERR_DEVICE.
 */
int sad_topk_propagate_rec(const float *rec, int sel_fmt, const uint32_t *scr, int n_slots, const uint32_t *cand_in,
                           uint32_t *cand_out, int W, int H, int cell, int jump, uint32_t pass_index, uint32_t seed,
                           int n_inject, void *stream);

/*
 * sad_render_fwd_rec -- sad_render_fwd from the site records (bit-identical when
 * they are current), on a map of any cell size: pixel (col, row) blends the list
 * of its entry, scored at its own centre ([SUM] B.3: the grid is looked up
 * without interpolation).
 *   rec device [n_slots][16]; cand device [Hm][Wm][8]; out_rgb device [H][W][3].
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_render_fwd_rec(const float *rec, int n_slots, const uint32_t *cand, int W, int H, int cell, float *out_rgb,
                       void *stream);

/*
 * sad_render_bwd_rec -- sad_render_bwd from the site records, on a map of any
 * cell size, into gradient records, with the loss spread over partial sums and
 * the forward image as a by-product:
 *   rec device [n_slots][16]; cand device [Hm][Wm][8]; target device [H][W][3];
 *   grad device [>= n_slots][16] float, +=, 16-byte aligned;
 *   loss_sum device float[SAD_LOSS_SLOTS] or NULL: each tile adds its sum of
 *   ||c - t||^2 to one of the entries (a thousand atomics on one address
 *   serialise); the loss is the entries' sum;
 *   out_rgb device [H][W][3] float or NULL: if given, the blend c(x) of every
 *   pixel is written there too -- the values sad_render_fwd_rec writes -- so a
 *   training step needs one pass over the map for forward and backward.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN (cand, rec or grad not 16-byte aligned),
 *         SAD_ERR_DEVICE.
 */
int sad_render_bwd_rec(const float *rec, int n_slots, const uint32_t *cand, const float *target, int W, int H,
                       int cell, float *grad, float *loss_sum, float *out_rgb, void *stream);

/*
 * sad_adam_step_rec -- sad_adam_step on gradient records (grad device
 * [stride][16], 16-byte aligned; words 0..9 zeroed, 10 left alone).  If rec is
 * not NULL the site records of slots [0, n_slots) are rewritten from the updated
 * sites in the same pass; if packed is not NULL, so are their packed words; if
 * scr is not NULL, so are their screen words (for the image cfg->x_max x
 * cfg->y_max).
 *   rec device [n_slots][16] or NULL; packed device [n_slots][4] uint32 or NULL,
 *   16-byte aligned; scr device [n_slots] uint32 or NULL; the rest as
 *   sad_adam_step.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_adam_step_rec(float *sites, float *m, float *v, float *grad, float *rec, uint32_t *packed, uint32_t *scr,
                      int n_slots, int stride, int step, int n_pixels, const sad_adam_cfg *cfg, void *stream);

/*
 * sad_densify_stats -- the budget-control statistics (see the rules above) on
 * the GPU, accumulated (+=) into `stats`.
 *   rec device [n_slots][16]; cand device [Hm][Wm][8]; target device [H][W][3];
 *   stats device [>= n_slots][SAD_STAT_LD] float, 16-byte aligned, +=.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_densify_stats(const float *rec, int n_slots, const uint32_t *cand, const float *target, int W, int H,
                      int cell, float *stats, void *stream);

/*
 * sad_densify_prune_stats -- rules 1-5 on the HOST, with statistics computed
 * elsewhere (sad_densify_stats) and a map of any cell size.  Seeding goes into
 * `cand` if it is not NULL, and as (entry index row*Wm + col, ID) pairs into
 * `seeds` if that is not NULL: grouped by entry (ascending) and in write order
 * within an entry, the form sad_apply_seeds takes.  The routine reads no list when
 * cand is NULL, so a caller whose map lives in device memory passes cand = NULL
 * and applies the pairs with sad_apply_seeds.  The removal accumulator is read,
 * not reset.
 *  sites [10][stride], m/v [10][stride], stats [stride][8], removal [stride],
 *  cand [Hm][Wm][8] or NULL, target [H][W][3] (all HOST); *n_slots in/out;
 *  n_split/n_pruned (out, may be NULL) receive the numbers of splits and prunes
 *  done; seeds uint32 [seeds_cap][2] or NULL with seeds_cap >= 5 * floor(split_frac
 *  * A) and *n_seeds (out) the number of pairs written.
 * Errors: SAD_ERR_ARG (checked before anything is modified, including a seeds
 *  buffer below that bound); SAD_ERR_CAPACITY as sad_densify_prune.
 */
int sad_densify_prune_stats(float *sites, float *m, float *v, int stride, int capacity, int *n_slots,
                            const float *stats, const float *removal, uint32_t *cand, int W, int H, int cell,
                            const float *target, const sad_budget_cfg *cfg, int *n_split, int *n_pruned,
                            uint32_t *seeds, long seeds_cap, long *n_seeds);

/*
 * sad_apply_seeds -- applies seeding pairs (entry, ID) from sad_densify_prune_stats
 * to a map in device memory, with rule 5: for each entry, its pairs in order,
 * each writes its ID into the last place of the entry's list unless the list
 * already holds it.  Pairs must be grouped by entry, in write order within an
 * entry (as sad_densify_prune_stats writes them); a pair whose entry lies
 * outside the map is skipped.
 *   cand device [Hm][Wm][8] (in/out, 16-byte aligned); seeds device uint32
 *   [n_seeds][2] (8-byte aligned); 0 <= n_seeds < 2^31.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_apply_seeds(uint32_t *cand, int W, int H, int cell, const uint32_t *seeds, long n_seeds, void *stream);

/* ======================================================================== */
/* Candidate-map tools                                                      */
/* ======================================================================== */

/*
 * sad_jfa_seed -- seed pass of the optional jump-flood prepass ([SUM] B.3 "Jump
 * schedule": a seed pass, then flood passes over 3x3 neighbourhoods that keep the
 * four closest sites; meant for (re)initialisation and after large edits).
 * Every active site with a finite position is entered in the list of the map
 * entry of the pixel that contains it (floor of its position, clamped into the
 * image); an entry keeps at most four, the best by (d, ID) at its centred UV, in
 * places 0..3 (ascending); all other places are SAD_INVALID.  The whole map is
 * written.
 *   rec/sel_fmt as in sad_topk_propagate_rec; cand device [Hm][Wm][8], written.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_jfa_seed(const float *rec, int sel_fmt, int n_slots, uint32_t *cand, int W, int H, int cell, void *stream);

/*
 * sad_jfa_pass -- one flood pass of the prepass with step `step` ([SUM] B.3):
 * per map entry, the union of places 0..3 of the lists at offsets {-step, 0,
 * step}^2 (in entries) that lie inside the map, without sentinels, IDs >=
 * n_slots, inactive sites, non-finite scores and duplicates; the four best by
 * (d, ID) at the entry's centred UV go to places 0..3 (ascending), SAD_INVALID to
 * 4..7.  Jacobi: reads cand_in, writes cand_out.  The prepass runs the steps B/2,
 * B/4, ..., 1 (B = 2^ceil(log2 max(Wm,Hm))), i.e. ceil(log2 max(Wm,Hm)) passes,
 * after sad_jfa_seed; propagation then fills the lists to K.
 *   rec/sel_fmt as in sad_topk_propagate_rec; step in [1, 65535]; cand_in,
 *   cand_out device [Hm][Wm][8], not overlapping.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_jfa_pass(const float *rec, int sel_fmt, int n_slots, const uint32_t *cand_in, uint32_t *cand_out, int W, int H,
                 int cell, int step, void *stream);

/*
 * sad_topk_exact -- the exact top-K map by brute force over every slot: the list
 * that propagation approximates ([NOTE] design 3; [SUM] section 4 "Candidate
 * maintenance").  Used to (re)initialise a map and to measure recall.  Cost
 * O(Wm*Hm*n_slots).  Same output convention as sad_topk_propagate.
 *   rec/sel_fmt as in sad_topk_propagate_rec;  cand_out device [Hm][Wm][8], written.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_topk_exact(const float *rec, int sel_fmt, int n_slots, uint32_t *cand_out, int W, int H, int cell,
                   void *stream);

/*
 * sad_topk_exact_at -- the exact top-K list (as sad_topk_exact) of chosen map
 * entries only, for recall measurements on maps where the whole-map brute force
 * is too costly.  Cost O(n_entries * n_slots).
 *   rec/sel_fmt as in sad_topk_propagate_rec;  entries device uint32 [n_entries],
 *   each a map entry index row*Wm + col (4-byte aligned); out device uint32
 *   [n_entries][8], written, 16-byte aligned.  An index outside the map gives an
 *   all-SAD_INVALID list.  0 <= n_entries.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_topk_exact_at(const float *rec, int sel_fmt, int n_slots, const uint32_t *entries, int n_entries, int W, int H,
                      int cell, uint32_t *out, void *stream);

/* ======================================================================== */
/* Evaluation format and random-access queries                              */
/* ======================================================================== */

/*
 * Evaluation format ([SUM] B.2 "Packed storage for evaluation": all ten values in
 * four 32-bit words, quantised, with per-image min/scale for log tau and r;
 * [PRESS] 5: 15-bit fixed-point coordinates, colour in 11/11/10 bits, 16 bits for
 * the temperature, the radius and the direction angle, float16 anisotropy):
 *   words [n_slots][4] uint32:
 *     w0 = qx | qy << 15 | inactive << 31      w1 = qR | qG << 11 | qB << 22
 *     w2 = q_logtau | q_r << 16                w3 = q_angle | f16(a) << 16
 *   header float[4] = {lt_min, lt_step, r_min, r_step}, step = (max - min)/65535
 *   over the active slots' finite values (0, 0 if none; a zero extreme is +0).
 * Codes: q = rint(t) (nearest even) clamped to [0, qmax], NaN -> 0, with t one
 * float32 product: x * (32767/W), y * (32767/H), R and G * 2047, B * 1023,
 * (log tau - lt_min) * (65535/(lt_max - lt_min)) (0 if max <= min), r likewise.
 * The direction is an axis (u and -u give one metric): theta = atan2(dy, dx) in
 * float64 folded into [0, pi), q = rint(theta * 65536/pi) mod 65536; 0 for a
 * degenerate direction (dx^2 + dy^2 < 1e-30).  a is IEEE binary16, nearest even.
 * An inactive slot (x < 0) is w0 = 1 << 31, w1 = w2 = w3 = 0.
 * Decoding (float32, each operation rounded on its own): x = qx * (W/32767),
 * y = qy * (H/32767), R = qR * (1/2047), G likewise, B = qB * (1/1023), log tau =
 * lt_min + q * lt_step, r = r_min + q * r_step, theta = q * (pi/65536), dir =
 * (cos theta, sin theta), a from binary16.
 */

/*
 * sad_eval_encode -- packs slots [0, n_slots) of `sites` into the evaluation
 * format: per-image ranges first, then one word quad per slot, then the header.
 *   sites device [10][stride] read-only; words device [n_slots][4] uint32, written,
 *   16-byte aligned; header device float[4], written (it holds the range keys
 *   while the call runs), 16-byte aligned.  W, H >= 1 (the position scale).
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_eval_encode(const float *sites, int n_slots, int stride, int W, int H, uint32_t *words, float *header,
                    void *stream);

/*
 * sad_eval_decode -- the site planes the evaluation words stand for (decoding
 * above); an inactive slot gets x = y = -1 and zeros.
 *   words device [n_slots][4] and header device float[4], read-only, 16-byte
 *   aligned; sites device [10][stride] float, slots [0, n_slots) written.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_eval_decode(const uint32_t *words, const float *header, int n_slots, int W, int H, float *sites, int stride,
                    void *stream);

/*
 * sad_eval_query -- random access ([SUM] abstract: fast random access; B.3
 * integer mapping of a position to its map entry).  Point i, (points[2i],
 * points[2i+1]) in pixels, reads the list of the map entry of the pixel that holds
 * it (coordinates clamped into the image) and is the softmax blend of those sites,
 * decoded from the evaluation words, evaluated at the point itself (the render's
 * score and blend; at a pixel centre it is that pixel's render).  A point with a
 * non-finite coordinate gives (0, 0, 0).
 *   words [n_slots][4], header float[4], cand [Hm][Wm][8] (16-byte aligned);
 *   points device float [n_points][2], 8-byte aligned; out_rgb device float
 *   [n_points][3], written.  0 <= n_points <= 2^31 - 256.
 * Errors: SAD_ERR_ARG, SAD_ERR_ALIGN, SAD_ERR_DEVICE.
 */
int sad_eval_query(const uint32_t *words, const float *header, int n_slots, const uint32_t *cand, int W, int H,
                   int cell, const float *points, int64_t n_points, float *out_rgb, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SAD_H */
