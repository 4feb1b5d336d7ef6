/*
 * sad_oracle.c -- plain CPU oracle for the Soft Anisotropic Diagrams (SAD) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library or its
 * Python binding) includes, links or calls this file; only the tests, the
 * package smoke check and the CPU-baseline leg of the benchmark do.  It shares
 * no code, header or constant with the GPU path.
 *
 * Sources (the pages):
 *   [SUM]  paperlayer.ai summary of arXiv:2604.21984v2 (sections 3-5, Appendix B)
 *   [NOTE] woaixuexisr.github.io reading note, "Key designs" 1-4 (the only explicit formulas)
 *   [PROJ] luckyiyi.github.io/SAD project page, "Method"
 *   [PRESS] 69574.cn article, sections 3-5
 *
 * Precision.  Everything that decides an integer (which site IDs a pixel keeps)
 * is computed in float32, the storage precision of the site buffer ([SUM] B.2),
 * so that the oracle and the GPU take that decision in the same precision; those
 * functions read float sites.  The render forward, backward and Adam read
 * float64 sites and compute in float64.
 * Compile with -ffp-contract=off: every operation below is rounded as written.
 *
 * Site buffer: ten float planes of `stride` entries, order
 *   x, y, log_tau, r, R, G, B, dir_x, dir_y, a     ([SUM] B.2; field list [PRESS] 5)
 * A slot with x < 0 is inactive ([SUM] B.2).  Candidate map: uint32 [H][W][8],
 * sentinel 0xffffffff ([SUM] B.2 "Top-K candidate list").
 *
 * Readings where the pages are open (each repeated at its function):
 *   - pixel (col,row) is evaluated at (col+0.5, row+0.5) px ([SUM] B.3, centred cells);
 *   - u = dir/|dir| (u = (1,0) when |dir|^2 < 1e-30), v = (-u_y, u_x);
 *   - candidates rank by (d ascending, site ID ascending);
 *   - injection: xorshift32 ([SUM] B.3 names xorshift) seeded by a PCG hash chain of
 *     (seed, pass word, pixel ID); IDs by multiply-shift range reduction;
 *   - an empty list renders 0; non-finite contributions are dropped.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_K 8
#define ORC_NONE 0xFFFFFFFFu
#define ORC_NPARAM 10
#define ORC_NACC 11
#define ORC_MAX_INJECT 16
#define ORC_MAX_UNION (5 * ORC_K + ORC_MAX_INJECT)

enum { P_X, P_Y, P_LOGTAU, P_R, P_CR, P_CG, P_CB, P_DX, P_DY, P_A };

static int g_threads = 1;

int orc_version(void) { return 1; }

void orc_set_threads(int n) { g_threads = n < 1 ? 1 : n; }

int orc_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------------ RNG --
 * [SUM] B.3 "Jump schedule": the pass word packs the step index (low 16 bits)
 * and the jump distance (high 16 bits); the xorshift state uses the step index
 * and the pixel ID.
 *
 * pcg_hash: the 32-bit "pcg" hash of Jarzynski & Olano, "Hash Functions for GPU
 * Rendering", JCGT 9(3), 2020 (one LCG step of PCG followed by the RXS-M-XS
 * output permutation).
 * xorshift32: Marsaglia, "Xorshift RNGs", J. Stat. Softw. 8(14), 2003, shifts (13,17,5).
 * Range reduction: Lemire, "Fast random integer generation in an interval",
 * ACM TOMACS 29(1), 2019 (multiply-shift, no rejection step).
 */
uint32_t orc_pcg_hash(uint32_t v)
{
    uint32_t state = v * 747796405u + 2891336453u;
    uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
    return (word >> 22u) ^ word;
}

uint32_t orc_xorshift32(uint32_t x)
{
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
}

uint32_t orc_pass_word(int jump, uint32_t pass_index)
{
    return ((uint32_t)jump << 16) | (pass_index & 0xFFFFu);
}

/* The M injected site IDs of one pixel in one pass (before any validity filter). */
void orc_inject_ids(uint32_t seed, int jump, uint32_t pass_index, uint32_t pix,
                    uint32_t n_slots, int m, uint32_t *out)
{
    uint32_t h = orc_pcg_hash(orc_pcg_hash(orc_pcg_hash(seed) ^ orc_pass_word(jump, pass_index)) ^ pix);
    uint32_t x = h ? h : 0x9E3779B9u; /* xorshift32 must not start at 0 */
    for (int j = 0; j < m; ++j) {
        x = orc_xorshift32(x);
        out[j] = (uint32_t)(((uint64_t)x * (uint64_t)n_slots) >> 32);
    }
}

/* --------------------------------------------------------------- score ---
 * [NOTE] design 1: G_i = e^{a} u u^T + e^{-a} v v^T (det G = 1),
 * d(x,i) = s*||x - p_i||_{G_i} - s*r_i with s = 1/max(H,W).
 * With alpha = u.delta and beta = v.delta, ||delta||_G = sqrt(e^a alpha^2 + e^-a beta^2).
 */
/* Candidate grid ([SUM] B.3 "Candidate field"): the map has ceil(W/c) x ceil(H/c)
 * cells, pixel (x, y) uses the list of cell (x/c, y/c) (integer division), and a
 * cell's candidates are selected at the cell centre in UV coordinates, which in
 * pixel units is ((cx + 1/2) W/Wm, (cy + 1/2) H/Hm).  c = 1 is the per-pixel map
 * (evaluation at pixel centres).  Reading: the pages give the grid size, the
 * integer mapping and the centred UVs, nothing more. */
typedef struct {
    int W, H, c, Wm, Hm;
    float sx, sy, s;
} grid;

static grid make_grid(int W, int H, int c)
{
    grid g;
    g.W = W;
    g.H = H;
    g.c = c < 1 ? 1 : c;
    g.Wm = (W + g.c - 1) / g.c;
    g.Hm = (H + g.c - 1) / g.c;
    g.sx = (float)W / (float)(g.Wm > 0 ? g.Wm : 1);
    g.sy = (float)H / (float)(g.Hm > 0 ? g.Hm : 1);
    g.s = 1.0f / (float)(W > H ? W : H);
    return g;
}

/* the map entry of pixel (col, row) */
static long cell_of(const grid *g, int col, int row) { return (long)(row / g->c) * g->Wm + col / g->c; }

static float score_at(const float *S, long stride, uint32_t id, float X, float Y, float s)
{
    float px = S[P_X * stride + id], py = S[P_Y * stride + id];
    float r = S[P_R * stride + id];
    float dx = S[P_DX * stride + id], dy = S[P_DY * stride + id];
    float a = S[P_A * stride + id];
    float ux = 1.0f, uy = 0.0f;
    float n2 = dx * dx + dy * dy;
    if (n2 >= 1e-30f) {
        float n = sqrtf(n2);
        ux = dx / n;
        uy = dy / n;
    }
    float vx = -uy, vy = ux;
    float ddx = X - px;
    float ddy = Y - py;
    float al = ux * ddx + uy * ddy;
    float be = vx * ddx + vy * ddy;
    float q = sqrtf(expf(a) * al * al + expf(-a) * be * be);
    return s * q - s * r;
}

/* selection score of map cell (cx, cy): evaluated at the cell's centred UV */
static float score_cell(const float *S, long stride, uint32_t id, const grid *g, int cx, int cy)
{
    return score_at(S, stride, id, ((float)cx + 0.5f) * g->sx, ((float)cy + 0.5f) * g->sy, g->s);
}


/* The same score in float64, with the intermediates the backward needs. */
typedef struct {
    double d, q, E, al, be, ux, uy, vx, vy, ddx, ddy, n;
    int degenerate_dir;
} geo64;

/* at the point (X, Y) px */
static void score_f64_at(const double *S, long stride, uint32_t id, double X, double Y, int W, int H, geo64 *g)
{
    double px = S[P_X * stride + id], py = S[P_Y * stride + id];
    double r = S[P_R * stride + id];
    double dx = S[P_DX * stride + id], dy = S[P_DY * stride + id];
    double a = S[P_A * stride + id];
    double s = 1.0 / (double)(W > H ? W : H);
    double n2 = dx * dx + dy * dy;
    g->ux = 1.0;
    g->uy = 0.0;
    g->n = 1.0;
    g->degenerate_dir = 1;
    if (n2 >= 1e-30) {
        g->n = sqrt(n2);
        g->ux = dx / g->n;
        g->uy = dy / g->n;
        g->degenerate_dir = 0;
    }
    g->vx = -g->uy;
    g->vy = g->ux;
    g->ddx = X - px;
    g->ddy = Y - py;
    g->al = g->ux * g->ddx + g->uy * g->ddy;
    g->be = g->vx * g->ddx + g->vy * g->ddy;
    g->E = exp(a);
    g->q = sqrt(g->E * g->al * g->al + g->be * g->be / g->E);
    g->d = s * g->q - s * r;
}

/* at the centre of pixel (col, row) */
static void score_f64(const double *S, long stride, uint32_t id, int col, int row, int W, int H, geo64 *g)
{
    score_f64_at(S, stride, id, (double)col + 0.5, (double)row + 0.5, W, H, g);
}

/* A list entry takes part if it names a slot below n_slots whose x (plane 0) is
 * not negative ([SUM] B.2: x < 0 marks an inactive site). */
static int site_usable(const float *S, uint32_t id, uint32_t n_slots)
{
    if (id == ORC_NONE || id >= n_slots)
        return 0;
    return !(S[id] < 0.0f);
}

static int site_usable64(const double *S, uint32_t id, uint32_t n_slots)
{
    if (id == ORC_NONE || id >= n_slots)
        return 0;
    return !(S[id] < 0.0);
}

/* Public: float32 selection scores of (pixel, id) pairs; unusable -> +inf. */
void orc_score_pairs(const float *S, int n_slots, int stride, int W, int H, int cell,
                     const uint32_t *pix, const uint32_t *ids, long n, float *out)
{
    grid g = make_grid(W, H, cell);
    for (long i = 0; i < n; ++i) {
        uint32_t id = ids[i];
        if (!site_usable(S, id, (uint32_t)n_slots)) {
            out[i] = INFINITY;
            continue;
        }
        float d = score_cell(S, stride, id, &g, (int)(pix[i] % (uint32_t)g.Wm), (int)(pix[i] / (uint32_t)g.Wm));
        out[i] = isfinite(d) ? d : INFINITY;
    }
}

/* Ranking key: (d ascending, ID ascending). */
static int key_less(float da, uint32_t ia, float db, uint32_t ib)
{
    return da < db || (da == db && ia < ib);
}

/* ----------------------------------------------------- exact top-K -------
 * The plain definition of the per-pixel top-K: score every active site and
 * keep the K best under (d, ID); pad with the sentinel.  ([NOTE] design 3:
 * the maintained list approximates the top-K under the same score.)
 */
static void exact_pixel(const float *S, uint32_t n_slots, long stride, const grid *g, int col, int row,
                        uint32_t *out)
{
    float bd[ORC_K];
    uint32_t bi[ORC_K];
    int cnt = 0;
    for (uint32_t id = 0; id < n_slots; ++id) {
        if (S[id] < 0.0f) /* inactive */
            continue;
        float d = score_cell(S, stride, id, g, col, row);
        if (!isfinite(d))
            continue;
        if (cnt == ORC_K && !key_less(d, id, bd[ORC_K - 1], bi[ORC_K - 1]))
            continue;
        int j = cnt < ORC_K ? cnt++ : ORC_K - 1;
        while (j > 0 && key_less(d, id, bd[j - 1], bi[j - 1])) {
            bd[j] = bd[j - 1];
            bi[j] = bi[j - 1];
            --j;
        }
        bd[j] = d;
        bi[j] = id;
    }
    for (int k = 0; k < ORC_K; ++k)
        out[k] = k < cnt ? bi[k] : ORC_NONE;
}

void orc_topk_exact(const float *S, int n_slots, int stride, int W, int H, int cell, uint32_t *cand)
{
    grid g = make_grid(W, H, cell);
    long P = (long)g.Wm * g.Hm;
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads)
    for (long p = 0; p < P; ++p)
        exact_pixel(S, (uint32_t)n_slots, stride, &g, (int)(p % g.Wm), (int)(p / g.Wm), cand + p * ORC_K);
}

void orc_topk_exact_pixels(const float *S, int n_slots, int stride, int W, int H, int cell,
                           const uint32_t *pix, long n, uint32_t *out)
{
    grid g = make_grid(W, H, cell);
#pragma omp parallel for schedule(dynamic, 16) num_threads(g_threads)
    for (long i = 0; i < n; ++i)
        exact_pixel(S, (uint32_t)n_slots, stride, &g, (int)(pix[i] % (uint32_t)g.Wm),
                    (int)(pix[i] / (uint32_t)g.Wm), out + i * ORC_K);
}

/* Hard (argmin) render: colour of the first entry of the exact top-K, 0 if none.
 * This is the temperature -> infinity limit of the blend ([NOTE] design 2). */
void orc_hard_render(const float *S, int n_slots, int stride, int W, int H, float *rgb)
{
    long P = (long)W * H;
    grid g = make_grid(W, H, 1);
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads)
    for (long p = 0; p < P; ++p) {
        uint32_t lst[ORC_K];
        exact_pixel(S, (uint32_t)n_slots, stride, &g, (int)(p % W), (int)(p / W), lst);
        for (int c = 0; c < 3; ++c)
            rgb[p * 3 + c] = lst[0] == ORC_NONE ? 0.0f : S[(P_CR + c) * (long)stride + lst[0]];
    }
}

/* -------------------------------------------------- propagation pass -----
 * [NOTE] design 3: C~_t(x) = C_{t-1}(x) U P_t(x) U G_t(x), then keep the top-K.
 *   C_{t-1}(x): the pixel's own list (temporal reuse);
 *   P_t(x):     the lists of the 4 neighbours at distance `jump` ([SUM] section 4,
 *               self-plus-4-neighbour propagation; neighbours outside the image are skipped);
 *   G_t(x):     n_inject IDs from the counter-based generator above.
 * Reading: a pass reads one map and writes another (Jacobi); sentinels, IDs
 * >= n_slots, inactive sites, non-finite scores and duplicates are removed.
 * The kept list is stored in ascending (d, ID) order, padded with the sentinel.
 */
static int union_pixel(const float *S, uint32_t n_slots, const uint32_t *cin, int W, int H, int col, int row,
                       int jump, uint32_t pass_index, uint32_t seed, int m, uint32_t *u)
{
    uint32_t raw[ORC_MAX_UNION];
    int nr = 0;
    const int ox[4] = {-jump, jump, 0, 0};
    const int oy[4] = {0, 0, -jump, jump};
    const uint32_t *own = cin + ((long)row * W + col) * ORC_K;
    for (int k = 0; k < ORC_K; ++k)
        raw[nr++] = own[k];
    for (int o = 0; o < 4; ++o) {
        int c = col + ox[o], r = row + oy[o];
        if (c < 0 || c >= W || r < 0 || r >= H)
            continue;
        const uint32_t *nb = cin + ((long)r * W + c) * ORC_K;
        for (int k = 0; k < ORC_K; ++k)
            raw[nr++] = nb[k];
    }
    orc_inject_ids(seed, jump, pass_index, (uint32_t)row * (uint32_t)W + (uint32_t)col, n_slots, m, raw + nr);
    nr += m;
    int nu = 0;
    for (int i = 0; i < nr; ++i) {
        uint32_t id = raw[i];
        if (!site_usable(S, id, n_slots))
            continue;
        int seen = 0;
        for (int j = 0; j < nu; ++j)
            if (u[j] == id)
                seen = 1;
        if (!seen)
            u[nu++] = id;
    }
    return nu;
}

/* (col, row): a cell of the map (a pixel when the grid's cell is 1); the union is
 * taken in map coordinates, the injection uses the cell's index. */
static void propagate_pixel(const float *S, uint32_t n_slots, long stride, const uint32_t *cin, const grid *g,
                            int col, int row, int jump, uint32_t pass_index, uint32_t seed, int m,
                            uint32_t *out)
{
    uint32_t u[ORC_MAX_UNION];
    float d[ORC_MAX_UNION];
    int nu = union_pixel(S, n_slots, cin, g->Wm, g->Hm, col, row, jump, pass_index, seed, m, u);
    int nv = 0;
    for (int i = 0; i < nu; ++i) {
        float di = score_cell(S, stride, u[i], g, col, row);
        if (!isfinite(di))
            continue;
        u[nv] = u[i];
        d[nv] = di;
        ++nv;
    }
    /* insertion sort by (d, ID) */
    for (int i = 1; i < nv; ++i) {
        float dk = d[i];
        uint32_t ik = u[i];
        int j = i;
        while (j > 0 && key_less(dk, ik, d[j - 1], u[j - 1])) {
            d[j] = d[j - 1];
            u[j] = u[j - 1];
            --j;
        }
        d[j] = dk;
        u[j] = ik;
    }
    for (int k = 0; k < ORC_K; ++k)
        out[k] = k < nv ? u[k] : ORC_NONE;
}

void orc_propagate(const float *S, int n_slots, int stride, const uint32_t *cin, uint32_t *cout, int W, int H,
                   int cell, int jump, uint32_t pass_index, uint32_t seed, int m)
{
    grid g = make_grid(W, H, cell);
    long P = (long)g.Wm * g.Hm;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long p = 0; p < P; ++p)
        propagate_pixel(S, (uint32_t)n_slots, stride, cin, &g, (int)(p % g.Wm), (int)(p / g.Wm), jump, pass_index,
                        seed, m, cout + p * ORC_K);
}

void orc_propagate_pixels(const float *S, int n_slots, int stride, const uint32_t *cin, int W, int H, int cell,
                          int jump, uint32_t pass_index, uint32_t seed, int m, const uint32_t *pix, long n,
                          uint32_t *out)
{
    grid g = make_grid(W, H, cell);
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long i = 0; i < n; ++i)
        propagate_pixel(S, (uint32_t)n_slots, stride, cin, &g, (int)(pix[i] % (uint32_t)g.Wm),
                        (int)(pix[i] / (uint32_t)g.Wm), jump, pass_index, seed, m, out + i * ORC_K);
}

/* The deduplicated, filtered candidate union of each listed pixel (for checking
 * that a GPU list only holds members of it).  out: n x ORC_MAX_UNION, count: n. */
void orc_union_pixels(const float *S, int n_slots, const uint32_t *cin, int W, int H, int cell, int jump,
                      uint32_t pass_index, uint32_t seed, int m, const uint32_t *pix, long n, uint32_t *out,
                      int *count)
{
    grid g = make_grid(W, H, cell);
    for (long i = 0; i < n; ++i) {
        uint32_t *u = out + i * ORC_MAX_UNION;
        int nu = union_pixel(S, (uint32_t)n_slots, cin, g.Wm, g.Hm, (int)(pix[i] % (uint32_t)g.Wm),
                             (int)(pix[i] / (uint32_t)g.Wm), jump, pass_index, seed, m, u);
        for (int j = nu; j < ORC_MAX_UNION; ++j)
            u[j] = ORC_NONE;
        count[i] = nu;
    }
}

int orc_max_union(void) { return ORC_MAX_UNION; }

/* ------------------------------------------------------ render forward ---
 * [NOTE] design 2 / [PROJ] "Method": l_i = -tau_i d_i, w = softmax over the
 * pixel's list, c(x) = sum_i w_i c_i; tau = exp(log_tau) ([PRESS] 6 quotes a
 * fixed log tau).  Max-subtracted softmax, invalid IDs skipped and non-finite
 * entries guarded ([SUM] B.4).  An empty list renders 0 (reading).
 */
typedef struct {
    int n;
    uint32_t id[ORC_K];
    geo64 g[ORC_K];
    double tau[ORC_K], l[ORC_K], w[ORC_K], e[ORC_K], c[ORC_K][3];
    double Z, chat[3];
} pix64;

/* The blend of list `lst` at the point (X, Y) px. */
static void forward_point(const double *S, uint32_t n_slots, long stride, const uint32_t *lst, int W, int H,
                          double X, double Y, pix64 *P)
{
    P->n = 0;
    for (int k = 0; k < ORC_K; ++k) {
        uint32_t id = lst[k];
        if (!site_usable64(S, id, n_slots))
            continue;
        int j = P->n;
        score_f64_at(S, stride, id, X, Y, W, H, &P->g[j]);
        double tau = exp(S[P_LOGTAU * stride + id]);
        double l = -tau * P->g[j].d;
        double c0 = S[P_CR * stride + id], c1 = S[P_CG * stride + id], c2 = S[P_CB * stride + id];
        if (!isfinite(l) || !isfinite(c0) || !isfinite(c1) || !isfinite(c2))
            continue;
        P->id[j] = id;
        P->tau[j] = tau;
        P->l[j] = l;
        P->c[j][0] = c0;
        P->c[j][1] = c1;
        P->c[j][2] = c2;
        P->n++;
    }
    P->chat[0] = P->chat[1] = P->chat[2] = 0.0;
    P->Z = 0.0;
    if (P->n == 0)
        return;
    double mx = P->l[0];
    for (int j = 1; j < P->n; ++j)
        if (P->l[j] > mx)
            mx = P->l[j];
    for (int j = 0; j < P->n; ++j) {
        P->e[j] = exp(P->l[j] - mx);
        P->Z += P->e[j];
    }
    for (int j = 0; j < P->n; ++j) {
        P->w[j] = P->e[j] / P->Z;
        for (int c = 0; c < 3; ++c)
            P->chat[c] += P->w[j] * P->c[j][c];
    }
}

/* The blend of pixel (col, row): at its centre. */
static void forward_pixel(const double *S, uint32_t n_slots, long stride, const uint32_t *lst, int W, int H,
                          int col, int row, pix64 *P)
{
    forward_point(S, n_slots, stride, lst, W, H, (double)col + 0.5, (double)row + 0.5, P);
}

/* Random-access query (the abstract's "fast random access"; [SUM] B.3 "Candidate
 * field": integer mapping of a position to its map entry).  Point i, (pts[2i],
 * pts[2i+1]) px, reads the list of the map entry of the pixel that holds it
 * (coordinates clamped into the image first) and is blended at the point itself.
 * A point with a non-finite coordinate returns (0, 0, 0). */
void orc_query_points(const double *S, int n_slots, int stride, const uint32_t *cand, int W, int H, int cell,
                      const float *pts, long n, double *rgb)
{
    grid g = make_grid(W, H, cell);
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long i = 0; i < n; ++i) {
        double X = pts[2 * i], Y = pts[2 * i + 1];
        rgb[3 * i] = rgb[3 * i + 1] = rgb[3 * i + 2] = 0.0;
        if (!isfinite(X) || !isfinite(Y))
            continue;
        double cx = X < 0.0 ? 0.0 : (X > (double)(W - 1) ? (double)(W - 1) : X);
        double cy = Y < 0.0 ? 0.0 : (Y > (double)(H - 1) ? (double)(H - 1) : Y);
        int col = (int)floor(cx), row = (int)floor(cy);
        pix64 P;
        forward_point(S, (uint32_t)n_slots, stride, cand + cell_of(&g, col, row) * ORC_K, W, H, X, Y, &P);
        for (int c = 0; c < 3; ++c)
            rgb[3 * i + c] = P.chat[c];
    }
}

void orc_render_fwd(const double *S, int n_slots, int stride, const uint32_t *cand, int W, int H, int cell,
                    double *rgb)
{
    grid g = make_grid(W, H, cell);
    long P = (long)W * H;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long p = 0; p < P; ++p) {
        pix64 X;
        int col = (int)(p % W), row = (int)(p / W);
        forward_pixel(S, (uint32_t)n_slots, stride, cand + cell_of(&g, col, row) * ORC_K, W, H, col, row, &X);
        for (int c = 0; c < 3; ++c)
            rgb[p * 3 + c] = X.chat[c];
    }
}

void orc_render_fwd_pixels(const double *S, int n_slots, int stride, const uint32_t *cand, int W, int H, int cell,
                           const uint32_t *pix, long n, double *rgb)
{
    grid g = make_grid(W, H, cell);
    for (long i = 0; i < n; ++i) {
        pix64 X;
        int col = (int)(pix[i] % (uint32_t)W), row = (int)(pix[i] / (uint32_t)W);
        forward_pixel(S, (uint32_t)n_slots, stride, cand + cell_of(&g, col, row) * ORC_K, W, H, col, row, &X);
        for (int c = 0; c < 3; ++c)
            rgb[i * 3 + c] = X.chat[c];
    }
}

/* ----------------------------------------------------- render backward ---
 * Hand-derived gradients of L = sum_x ||c(x) - t(x)||^2 (un-normalised; Adam
 * divides by the pixel count, [SUM] B.4) with the map held fixed.  Per pixel,
 * g = 2 (c - t); per valid entry k ([SUM] B.4 lists the parameters):
 *   dL/dc_k      = w_k g
 *   gamma_k      = dL/dl_k = w_k g.(c_k - c)
 *   dL/dlog_tau  = gamma_k l_k                      (l = -exp(log_tau) d)
 *   dL/dd_k      = -tau_k gamma_k
 *   dL/dr        = tau_k gamma_k s                  (d = s q - s r)
 *   eta          = dL/dq = -tau_k gamma_k s;  q^2 = E al^2 + be^2/E, E = e^a
 *   dL/da        = eta (E al^2 - be^2/E) / (2q)
 *   dL/dp        = -(eta/q) (E al u + (be/E) v)
 *   dL/du        = (eta/q) (E al delta + (be/E) (delta_y, -delta_x)),
 *   dL/ddir      = (I - u u^T) dL/du / |dir|        (u = dir/|dir|)
 * With q = 0 the p, a and dir terms are 0 (subgradient); with a degenerate
 * dir the dir term is 0.  Accumulator 10 is the removal delta ([SUM] B.4-B.5):
 *   Delta_k = ||c_{-k} - t||^2 - ||c - t||^2, c_{-k} the blend of the other
 *   entries renormalised (0 if they carry no weight).
 * Non-finite contributions are dropped ([SUM] B.4: the NaN guard).
 * Accumulation is in float64 (orc_render_bwd states the order).
 */
static void backward_pixel(long stride, int W, int H, const pix64 *X, const float *t,
                           double *grad, double *loss)
{
    if (X->n == 0) {
        double e0 = 0.0;
        for (int c = 0; c < 3; ++c)
            e0 += (0.0 - t[c]) * (0.0 - t[c]);
        *loss += e0;
        return;
    }
    double s = 1.0 / (double)(W > H ? W : H);
    double gv[3], err = 0.0;
    for (int c = 0; c < 3; ++c) {
        double r = X->chat[c] - (double)t[c];
        gv[c] = 2.0 * r;
        err += r * r;
    }
    *loss += err;
    for (int k = 0; k < X->n; ++k) {
        const geo64 *G = &X->g[k];
        double w = X->w[k];
        double acc[ORC_NACC];
        memset(acc, 0, sizeof(acc));
        double gamma = 0.0;
        for (int c = 0; c < 3; ++c) {
            acc[P_CR + c] = w * gv[c];
            gamma += gv[c] * (X->c[k][c] - X->chat[c]);
        }
        gamma *= w;
        acc[P_LOGTAU] = gamma * X->l[k];
        acc[P_R] = X->tau[k] * gamma * s;
        double eta = -X->tau[k] * gamma * s;
        if (G->q > 0.0) {
            double E = G->E, iE = 1.0 / G->E;
            double f = eta / G->q;
            acc[P_X] = -f * (E * G->al * G->ux + iE * G->be * G->vx);
            acc[P_Y] = -f * (E * G->al * G->uy + iE * G->be * G->vy);
            acc[P_A] = eta * (E * G->al * G->al - iE * G->be * G->be) / (2.0 * G->q);
            if (!G->degenerate_dir) {
                double gux = f * (E * G->al * G->ddx + iE * G->be * G->ddy);
                double guy = f * (E * G->al * G->ddy - iE * G->be * G->ddx);
                double proj = G->ux * gux + G->uy * guy;
                acc[P_DX] = (gux - proj * G->ux) / G->n;
                acc[P_DY] = (guy - proj * G->uy) / G->n;
            }
        }
        /* removal delta: renormalise the other entries directly */
        double Zo = 0.0, co[3] = {0.0, 0.0, 0.0};
        for (int j = 0; j < X->n; ++j) {
            if (j == k)
                continue;
            Zo += X->e[j];
            for (int c = 0; c < 3; ++c)
                co[c] += X->e[j] * X->c[j][c];
        }
        double err_o = 0.0;
        for (int c = 0; c < 3; ++c) {
            double cm = Zo > 0.0 ? co[c] / Zo : 0.0;
            double r = cm - (double)t[c];
            err_o += r * r;
        }
        acc[10] = err_o - err;
        uint32_t id = X->id[k];
        for (int a = 0; a < ORC_NACC; ++a)
            if (isfinite(acc[a]))
                grad[(long)a * stride + id] += acc[a];
    }
}

/* grad: float64 [11][stride], accumulated (+=).  loss: += sum_x ||c - t||^2.
 * The image is cut into as many bands of whole rows as there are threads; each
 * band sums its pixels in pixel order into its own accumulators (band 0 into
 * grad itself), and the bands are then added to grad in band order.  With one
 * thread this is the serial sum in pixel order. */
void orc_render_bwd(const double *S, int n_slots, int stride, const uint32_t *cand, const float *target, int W,
                    int H, int cell, double *grad, double *loss)
{
    grid g = make_grid(W, H, cell);
    int nb = g_threads < H ? g_threads : H;
    if (nb < 1)
        nb = 1;
    long plane = (long)ORC_NACC * stride;
    double *priv = nb > 1 ? calloc((size_t)(nb - 1) * plane, sizeof(double)) : NULL;
    if (nb > 1 && !priv)
        nb = 1;  /* no memory for the band accumulators: one band */
    double *Lb = calloc((size_t)nb, sizeof(double));
#pragma omp parallel for schedule(static, 1) num_threads(nb)
    for (int b = 0; b < nb; ++b) {
        double *gb = b == 0 ? grad : priv + (long)(b - 1) * plane;
        long p0 = (long)W * (long)((long)H * b / nb), p1 = (long)W * (long)((long)H * (b + 1) / nb);
        for (long p = p0; p < p1; ++p) {
            pix64 X;
            int col = (int)(p % W), row = (int)(p / W);
            forward_pixel(S, (uint32_t)n_slots, stride, cand + cell_of(&g, col, row) * ORC_K, W, H, col, row, &X);
            backward_pixel(stride, W, H, &X, target + p * 3, gb, &Lb[b]);
        }
    }
    double L = 0.0;
    for (int b = 0; b < nb; ++b)
        L += Lb[b];
    if (nb > 1) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
        for (long o = 0; o < plane; ++o)
            for (int b = 1; b < nb; ++b)
                grad[o] += priv[(long)(b - 1) * plane + o];
    }
    free(priv);
    free(Lb);
    if (loss)
        *loss += L;
}

/* ------------------------------------------------------------- Adam ------
 * Adam (Kingma & Ba, ICLR 2015) on the ten site parameters ([SUM] sections 4-5,
 * B.4: accumulators are divided by the pixel count).  Per active slot (x >= 0)
 * and parameter j:  g = G_j / P (non-finite -> 0);  m = b1 m + (1-b1) g;
 * v = b2 v + (1-b2) g^2;  theta -= lr_j (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps).
 * Then x is clamped to [0, W] and y to [0, H] (reading: keeps a moving site from
 * crossing into the x < 0 "inactive" marker).  Gradient planes 0..9 of every
 * slot below n_slots are zeroed; plane 10 (removal delta) is left alone.
 * Arrays are float64 here: params/m/v [10][stride], grad [11][stride].
 */
void orc_adam_step(double *params, double *m, double *v, double *grad, int n_slots, int stride, int step,
                   int n_pixels, const double *lr, double b1, double b2, double eps, int W, int H)
{
    double bc1 = 1.0 - pow(b1, (double)step);
    double bc2 = 1.0 - pow(b2, (double)step);
    /* slots are independent */
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long i = 0; i < n_slots; ++i) {
        if (!(params[i] < 0.0)) {
            for (int j = 0; j < ORC_NPARAM; ++j) {
                long o = (long)j * stride + i;
                double g = grad[o] / (double)n_pixels;
                if (!isfinite(g))
                    g = 0.0;
                m[o] = b1 * m[o] + (1.0 - b1) * g;
                v[o] = b2 * v[o] + (1.0 - b2) * g * g;
                double mh = m[o] / bc1;
                double vh = v[o] / bc2;
                params[o] -= lr[j] * mh / (sqrt(vh) + eps);
            }
            double *x = &params[(long)P_X * stride + i], *y = &params[(long)P_Y * stride + i];
            *x = *x < 0.0 ? 0.0 : (*x > W ? (double)W : *x);
            *y = *y < 0.0 ? 0.0 : (*y > H ? (double)H : *y);
        }
        for (int j = 0; j < ORC_NPARAM; ++j)
            grad[(long)j * stride + i] = 0.0;
    }
}

/* --------------------------------------------------- budget statistics -----
 * [SUM] B.5: a site's claim to be split is judged from how much image it
 * covers, how much error it leaves and how that error is spread (its
 * error-weighted second moments).  Per site i, over the pixels x whose list holds it
 * (w = its softmax weight at x, e = ||c(x) - t(x)||^2, delta = x - p_i):
 *   [0] sum w  [1] sum w e  [2] sum w e dx  [3] sum w e dy
 *   [4] sum w e dx^2  [5] sum w e dx dy  [6] sum w e dy^2  [7] unused
 * stats: float64 [stride][8], accumulated (+=), serial in pixel order.
 */
void orc_densify_stats(const double *S, int n_slots, int stride, const uint32_t *cand, const float *target, int W,
                       int H, int cell, double *stats)
{
    grid g = make_grid(W, H, cell);
    long P = (long)W * H;
    for (long p = 0; p < P; ++p) {
        pix64 X;
        int col = (int)(p % W), row = (int)(p / W);
        forward_pixel(S, (uint32_t)n_slots, stride, cand + cell_of(&g, col, row) * ORC_K, W, H, col, row, &X);
        if (X.n == 0)
            continue;
        double e = 0.0;
        for (int c = 0; c < 3; ++c) {
            double r = X.chat[c] - (double)target[p * 3 + c];
            e += r * r;
        }
        for (int k = 0; k < X.n; ++k) {
            double w = X.w[k], we = w * e;
            double dx = ((double)col + 0.5) - S[(long)P_X * stride + X.id[k]];
            double dy = ((double)row + 0.5) - S[(long)P_Y * stride + X.id[k]];
            double *o = stats + (long)X.id[k] * 8;
            o[0] += w;
            o[1] += we;
            o[2] += we * dx;
            o[3] += we * dy;
            o[4] += we * dx * dx;
            o[5] += we * dx * dy;
            o[6] += we * dy * dy;
        }
    }
}

/* ------------------------------------------------------ JFA prepass ------
 * [SUM] B.3 "Jump schedule": an optional jump-flood prepass for
 * (re)initialisation -- a seed pass, then ceil(log2 max(W,H)) flood passes that
 * sample 3x3 neighbourhoods and write the four closest sites.
 * Readings (the pages give no more): the seed pass puts each active site with a
 * finite position into the list of the pixel that contains it (the floor of its
 * position, clamped into the image); a pixel keeps at most four of them, the
 * best by (d, ID) at its centre.  A flood pass with step k takes, per pixel, the
 * union of the first four entries of the lists at the offsets {-k, 0, k}^2 that
 * lie inside the image, drops sentinels, IDs >= n_slots, inactive sites,
 * non-finite scores and duplicates, and keeps the four best by (d, ID) in
 * entries 0..3; entries 4..7 hold the sentinel.  A pass reads one map and writes
 * another.  Selection runs in float32 like the propagation's.
 */
#define ORC_JFA_KEEP 4
#define ORC_JFA_UNION (9 * ORC_JFA_KEEP)

static void sort_by_score(float *d, uint32_t *u, int n)
{
    for (int i = 1; i < n; ++i) {
        float dk = d[i];
        uint32_t ik = u[i];
        int j = i;
        while (j > 0 && key_less(dk, ik, d[j - 1], u[j - 1])) {
            d[j] = d[j - 1];
            u[j] = u[j - 1];
            --j;
        }
        d[j] = dk;
        u[j] = ik;
    }
}

void orc_jfa_seed(const float *S, int n_slots, int stride, int W, int H, int cell, uint32_t *cand)
{
    grid g = make_grid(W, H, cell);
    long P = (long)g.Wm * g.Hm;
    for (long i = 0; i < P * ORC_K; ++i)
        cand[i] = ORC_NONE;
    for (uint32_t id = 0; id < (uint32_t)n_slots; ++id) {
        if (!site_usable(S, id, (uint32_t)n_slots))
            continue;
        float x = S[id], y = S[(long)stride + id];
        if (!isfinite(x) || !isfinite(y))
            continue;
        /* the pixel that contains the site, clamped into the image (in float first,
         * so that any finite position converts) */
        float cx = x < 0.0f ? 0.0f : (x > (float)(W - 1) ? (float)(W - 1) : x);
        float cy = y < 0.0f ? 0.0f : (y > (float)(H - 1) ? (float)(H - 1) : y);
        int col = (int)floorf(cx) / g.c, row = (int)floorf(cy) / g.c; /* its cell */
        float d = score_cell(S, stride, id, &g, col, row);
        if (!isfinite(d))
            continue;
        uint32_t *lst = cand + ((long)row * g.Wm + col) * ORC_K;
        float dd[ORC_JFA_KEEP + 1];
        uint32_t uu[ORC_JFA_KEEP + 1];
        int n = 0;
        for (int k = 0; k < ORC_JFA_KEEP && lst[k] != ORC_NONE; ++k) {
            uu[n] = lst[k];
            dd[n] = score_cell(S, stride, lst[k], &g, col, row);
            ++n;
        }
        uu[n] = id;
        dd[n] = d;
        ++n;
        sort_by_score(dd, uu, n);
        for (int k = 0; k < ORC_JFA_KEEP; ++k)
            lst[k] = k < n ? uu[k] : ORC_NONE;
    }
}

static int jfa_union_pixel(const float *S, uint32_t n_slots, const uint32_t *cin, int W, int H, int col, int row,
                           int step, uint32_t *u)
{
    int nu = 0;
    for (int dy = -1; dy <= 1; ++dy)
        for (int dx = -1; dx <= 1; ++dx) {
            int c = col + dx * step, r = row + dy * step;
            if (c < 0 || c >= W || r < 0 || r >= H)
                continue;
            const uint32_t *lst = cin + ((long)r * W + c) * ORC_K;
            for (int k = 0; k < ORC_JFA_KEEP; ++k) {
                uint32_t id = lst[k];
                if (!site_usable(S, id, n_slots))
                    continue;
                int seen = 0;
                for (int j = 0; j < nu; ++j)
                    if (u[j] == id)
                        seen = 1;
                if (!seen)
                    u[nu++] = id;
            }
        }
    return nu;
}

static void jfa_pixel(const float *S, uint32_t n_slots, long stride, const uint32_t *cin, const grid *g, int col,
                      int row, int step, uint32_t *out)
{
    uint32_t u[ORC_JFA_UNION];
    float d[ORC_JFA_UNION];
    int nu = jfa_union_pixel(S, n_slots, cin, g->Wm, g->Hm, col, row, step, u);
    int nv = 0;
    for (int i = 0; i < nu; ++i) {
        float di = score_cell(S, stride, u[i], g, col, row);
        if (!isfinite(di))
            continue;
        u[nv] = u[i];
        d[nv] = di;
        ++nv;
    }
    sort_by_score(d, u, nv);
    for (int k = 0; k < ORC_K; ++k)
        out[k] = (k < ORC_JFA_KEEP && k < nv) ? u[k] : ORC_NONE;
}

void orc_jfa_pass(const float *S, int n_slots, int stride, const uint32_t *cin, uint32_t *cout, int W, int H,
                  int cell, int step)
{
    grid g = make_grid(W, H, cell);
    long P = (long)g.Wm * g.Hm;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long p = 0; p < P; ++p)
        jfa_pixel(S, (uint32_t)n_slots, stride, cin, &g, (int)(p % g.Wm), (int)(p / g.Wm), step, cout + p * ORC_K);
}

void orc_jfa_pass_pixels(const float *S, int n_slots, int stride, const uint32_t *cin, int W, int H, int cell,
                         int step, const uint32_t *pix, long n, uint32_t *out)
{
    grid g = make_grid(W, H, cell);
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long i = 0; i < n; ++i)
        jfa_pixel(S, (uint32_t)n_slots, stride, cin, &g, (int)(pix[i] % (uint32_t)g.Wm),
                  (int)(pix[i] / (uint32_t)g.Wm), step, out + i * ORC_K);
}

/* The deduplicated union a flood pass selects from (padded to ORC_MAX_UNION). */
void orc_jfa_union_pixels(const float *S, int n_slots, const uint32_t *cin, int W, int H, int cell, int step,
                          const uint32_t *pix, long n, uint32_t *out, int *count)
{
    grid g = make_grid(W, H, cell);
    for (long i = 0; i < n; ++i) {
        uint32_t u[ORC_JFA_UNION];
        int nu = jfa_union_pixel(S, (uint32_t)n_slots, cin, g.Wm, g.Hm, (int)(pix[i] % (uint32_t)g.Wm),
                                 (int)(pix[i] / (uint32_t)g.Wm), step, u);
        for (int j = 0; j < ORC_MAX_UNION; ++j)
            out[i * ORC_MAX_UNION + j] = j < nu ? u[j] : ORC_NONE;
        count[i] = nu;
    }
}
