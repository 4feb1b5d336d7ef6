// sad_budget.cpp -- host-side budget control (densify / prune) of libsad.
//
// The rules follow the paperlayer.ai summary, Appendix B.5: sites are ranked for
// splitting by their error energy over a power of their mass, a split places two
// children along an axis taken from the error-weighted covariance (or, without
// enough mass, from the local luminance gradient), the children copy the parent
// with their colour read from the target, shrunken r and log tau and fresh Adam
// moments; pruning drops the sites whose removal would raise the error least and
// marks them with position (-1, -1).  Also the reading note's key design 4 and
// the press article's section 4.  The statistics come from sad_densify_stats on
// the GPU (sad_densify_prune_stats) or from host_stats below (sad_densify_prune).
// Readings where the pages are silent are stated in include/sad.h.

#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <numeric>
#include <system_error>
#include <thread>
#include <vector>

#include "sad.h"

namespace {

enum { PX, PY, PLT, PR, PCR, PCG, PCB, PDX, PDY, PA };

struct Img {
    const float *t;
    int W, H;
    float lum(int c, int r) const
    {
        c = std::min(std::max(c, 0), W - 1);
        r = std::min(std::max(r, 0), H - 1);
        const float *q = t + 3 * ((long)r * W + c);
        return 0.299f * q[0] + 0.587f * q[1] + 0.114f * q[2];
    }
    int col(double x) const { return std::min(std::max((int)std::floor(x), 0), W - 1); }
    int row(double y) const { return std::min(std::max((int)std::floor(y), 0), H - 1); }
};

// Principal axis of the 2x2 symmetric matrix [[a, b], [b, c]].
void principal_axis(double a, double b, double c, double &lam, double &ex, double &ey)
{
    const double h = 0.5 * (a - c);
    lam = 0.5 * (a + c) + std::sqrt(h * h + b * b);
    if (std::fabs(b) > 1e-300) {
        ex = lam - c;
        ey = b;
    } else {
        ex = a >= c ? 1.0 : 0.0;
        ey = a >= c ? 0.0 : 1.0;
    }
    const double n = std::sqrt(ex * ex + ey * ey);
    ex /= n;
    ey /= n;
}

// Runs f(lo, hi) over [0, n) in contiguous ranges on up to 8 host threads (the
// calling thread takes the first range); fewer threads for small n, and the
// calling thread alone if threads cannot be started.  The ranges write disjoint
// data, so the result does not depend on the thread count.
template <class F>
void parallel_for(long n, F f)
{
    const long hw = (long)std::max(1u, std::thread::hardware_concurrency());
    const long T = std::max(1L, std::min({hw, 8L, n / 2048}));
    std::vector<std::thread> th;
    long started = 1;
    try {
        for (long t = 1; t < T; ++t, ++started)
            th.emplace_back(f, n * t / T, n * (t + 1) / T);
    } catch (const std::system_error &) {
    }
    f(0, n / T);
    for (long t = started; t < T; ++t)  // the ranges no thread took
        f(n * t / T, n * (t + 1) / T);
    for (auto &x : th)
        x.join();
}

// The budget-control statistics of include/sad.h on the host, in float64, over
// the per-pixel map: per pixel the softmax blend of its list (usable entries: an
// ID below n of an active site with a finite logit and colour; a duplicate ID
// counts twice, as in the render), e = ||c - t||^2, then for each usable entry
// with w > 0 the seven sums.  Rows are split over up to 8 threads with their own
// accumulators, added in thread order.
void host_stats(const float *sites, int n, long st, const uint32_t *cand, int W, int H, const float *target,
                float *stats)
{
    const double s = 1.0 / (double)std::max(W, H);
    const long hw = (long)std::max(1u, std::thread::hardware_concurrency());
    const int T = (int)std::max(1L, std::min({hw, 8L, (long)H / 16}));
    std::vector<std::vector<double>> acc(T);
    auto rows = [&](int t) {
        std::vector<double> &a = acc[t];
        a.assign((size_t)n * 7, 0.0);
        const int r0 = (int)((long)H * t / T), r1 = (int)((long)H * (t + 1) / T);
        for (int row = r0; row < r1; ++row)
            for (int col = 0; col < W; ++col) {
                const long p = (long)row * W + col;
                const double X = col + 0.5, Y = row + 0.5;
                double l[SAD_K], cr[SAD_K][3];
                int id[SAD_K];
                bool use[SAD_K];
                double lmax = -INFINITY;
                for (int k = 0; k < SAD_K; ++k) {
                    const uint32_t c = cand[p * SAD_K + k];
                    use[k] = false;
                    id[k] = (int)c;
                    if (c >= (uint32_t)n || sites[PX * st + c] < 0.0f)
                        continue;
                    const double px = sites[PX * st + c], py = sites[PY * st + c];
                    double ux = sites[PDX * st + c], uy = sites[PDY * st + c];
                    const double n2 = ux * ux + uy * uy;
                    if (n2 < 1e-30) {
                        ux = 1.0;
                        uy = 0.0;
                    } else {
                        const double in = 1.0 / std::sqrt(n2);
                        ux *= in;
                        uy *= in;
                    }
                    const double a = sites[PA * st + c];
                    const double dx = X - px, dy = Y - py;
                    const double al = ux * dx + uy * dy, be = ux * dy - uy * dx;
                    const double q = std::sqrt(std::exp(a) * al * al + std::exp(-a) * be * be);
                    const double d = s * q - s * (double)sites[PR * st + c];
                    l[k] = -std::exp((double)sites[PLT * st + c]) * d;
                    for (int ch = 0; ch < 3; ++ch)
                        cr[k][ch] = sites[(PCR + ch) * st + c];
                    use[k] = std::isfinite(l[k]) && std::isfinite(cr[k][0]) && std::isfinite(cr[k][1]) &&
                             std::isfinite(cr[k][2]);
                    if (use[k])
                        lmax = std::max(lmax, l[k]);
                }
                if (!(lmax > -INFINITY))
                    continue;
                double e[SAD_K], Z = 0.0, chat[3] = {0.0, 0.0, 0.0};
                for (int k = 0; k < SAD_K; ++k) {
                    e[k] = use[k] ? std::exp(l[k] - lmax) : 0.0;
                    Z += e[k];
                }
                for (int k = 0; k < SAD_K; ++k)
                    for (int ch = 0; ch < 3; ++ch)
                        chat[ch] += use[k] ? e[k] / Z * cr[k][ch] : 0.0;
                const float *tp = target + 3 * p;
                const double err = (chat[0] - tp[0]) * (chat[0] - tp[0]) + (chat[1] - tp[1]) * (chat[1] - tp[1]) +
                                   (chat[2] - tp[2]) * (chat[2] - tp[2]);
                for (int k = 0; k < SAD_K; ++k) {
                    const double w = e[k] / Z;
                    if (!use[k] || !(w > 0.0))
                        continue;
                    const int c = id[k];
                    const double dx = X - sites[PX * st + c], dy = Y - sites[PY * st + c], we = w * err;
                    const double v7[7] = {w, we, we * dx, we * dy, we * dx * dx, we * dx * dy, we * dy * dy};
                    for (int j = 0; j < 7; ++j)
                        if (std::isfinite(v7[j]))
                            a[(size_t)c * 7 + j] += v7[j];
                }
            }
    };
    std::vector<std::thread> th;
    int started = 1;
    try {
        for (int t = 1; t < T; ++t, ++started)
            th.emplace_back(rows, t);
    } catch (const std::system_error &) {
    }
    rows(0);
    for (int t = started; t < T; ++t)
        rows(t);
    for (auto &x : th)
        x.join();
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < 7; ++j) {
            double v = 0.0;
            for (int t = 0; t < T; ++t)
                v += acc[t][(size_t)i * 7 + j];
            stats[(size_t)i * SAD_STAT_LD + j] = (float)v;
        }
        stats[(size_t)i * SAD_STAT_LD + 7] = 0.0f;
    }
}

}  // namespace

extern "C" int sad_densify_prune_stats(float *sites, float *m, float *v, int stride, int capacity, int *n_slots,
                                       const float *stats, const float *removal, uint32_t *cand, int W, int H,
                                       int cell, const float *target, const sad_budget_cfg *cfg, int *n_split_out,
                                       int *n_pruned_out, uint32_t *seeds, long seeds_cap, long *n_seeds_out)
{
    if (!sites || !m || !v || !n_slots || !stats || !removal || !target || !cfg)
        return SAD_ERR_ARG;
    const int n = *n_slots;
    if (n < 0 || stride < 1 || n > stride || capacity < n || capacity > stride || W < 1 || H < 1 ||
        W > SAD_MAX_DIM || H > SAD_MAX_DIM || cell < 1 || cell > SAD_MAX_DIM)
        return SAD_ERR_ARG;
    const int Wm = (W + cell - 1) / cell, Hm = (H + cell - 1) / cell;
    if (!(cfg->split_frac >= 0.0f && cfg->split_frac <= 1.0f && cfg->prune_frac >= 0.0f &&
          cfg->prune_frac <= 1.0f && cfg->shrink > 0.0f && cfg->min_mass >= 0.0f))
        return SAD_ERR_ARG;
    const long st = stride;
    auto P = [&](int j, int i) -> float & { return sites[j * st + i]; };

    std::vector<int> active;
    for (int i = 0; i < n; ++i)
        if (!(P(PX, i) < 0.0f))
            active.push_back(i);
    const long A = (long)active.size();
    const int n_split = (int)std::floor((double)cfg->split_frac * (double)A);
    // every split seeds at most five map entries
    if (seeds && (seeds_cap < 5L * n_split || !n_seeds_out))
        return SAD_ERR_ARG;
    long n_seeds = 0;
    const int n_prune = (int)std::floor((double)cfg->prune_frac * (double)A);

    // 1. split set: largest score, ties -> lower ID.  Only the first n_split in
    // that order are needed, and in that order (it decides which free slot each
    // second child takes): select them, then sort the selection.
    std::vector<double> score(active.size());
    parallel_for((long)active.size(), [&](long lo, long hi) {
        for (long j = lo; j < hi; ++j) {
            const long i = active[j];
            const double mass = stats[i * SAD_STAT_LD + 0], energy = stats[i * SAD_STAT_LD + 1];
            score[j] = energy / std::pow(std::max(mass, (double)cfg->min_mass), (double)cfg->alpha);
        }
    });
    std::vector<std::pair<double, int>> sc;
    sc.reserve(active.size());
    for (size_t j = 0; j < active.size(); ++j)
        if (std::isfinite(score[j]) && score[j] > 0.0)
            sc.push_back({score[j], active[j]});
    const auto split_first = [](const std::pair<double, int> &a, const std::pair<double, int> &b) {
        return a.first > b.first || (a.first == b.first && a.second < b.second);
    };
    const size_t k_split = std::min(sc.size(), (size_t)n_split);
    if (k_split < sc.size())
        std::nth_element(sc.begin(), sc.begin() + k_split, sc.end(), split_first);
    std::sort(sc.begin(), sc.begin() + k_split, split_first);
    std::vector<int> split;
    split.reserve(k_split);
    for (size_t j = 0; j < k_split; ++j)
        split.push_back(sc[j].second);
    std::vector<char> is_split(n, 0);
    for (int i : split)
        is_split[i] = 1;

    // 2. prune set: smallest removal delta among the others, ties -> lower ID
    // (a set: the order of pruning changes nothing)
    std::vector<std::pair<double, int>> rm;
    rm.reserve(active.size());
    for (int i : active)
        if (!is_split[i] && std::isfinite(removal[i]))
            rm.push_back({(double)removal[i], i});
    const size_t k_prune = std::min(rm.size(), (size_t)std::max(n_prune, 0));
    if (k_prune < rm.size())
        std::nth_element(rm.begin(), rm.begin() + k_prune, rm.end(),
                         [](const std::pair<double, int> &a, const std::pair<double, int> &b) {
                             return a.first < b.first || (a.first == b.first && a.second < b.second);
                         });
    const int pruned = (int)k_prune;
    parallel_for((long)k_prune, [&](long lo, long hi) {
        for (long j = lo; j < hi; ++j) {
            const int i = rm[j].second;
            P(PX, i) = -1.0f;
            P(PY, i) = -1.0f;
            for (int q = 0; q < SAD_NPARAM; ++q)
                m[q * st + i] = v[q * st + i] = 0.0f;
        }
    });

    // free slots for the second children: inactive slots below n (ascending), then n, n+1, ...
    std::vector<int> free_slots;
    for (int i = 0; i < n; ++i)
        if (P(PX, i) < 0.0f)
            free_slots.push_back(i);
    size_t next_free = 0;
    int count = n;
    auto take_slot = [&]() -> int {
        if (next_free < free_slots.size())
            return free_slots[next_free++];
        if (count < capacity)
            return count++;
        return -1;
    };

    // 3. splits.  The second children's slots are assigned in split order (the
    // first split that finds none ends the splitting); the splits then write
    // disjoint slots (a parent's own and its second child's) and run in parallel;
    // the map entries they seed are applied afterwards, in split order.
    const Img img{target, W, H};
    const float lshrink = std::log(cfg->shrink);
    std::vector<int> bslot;
    bslot.reserve(split.size());
    bool short_of_slots = false;
    for (size_t j = 0; j < split.size(); ++j) {
        const int b = take_slot();
        if (b < 0) {
            short_of_slots = true;
            break;
        }
        bslot.push_back(b);
    }
    const int done = (int)bslot.size();
    std::vector<long> seed_e((size_t)done * 5, -1L);  // per split: seeded entries, -1 = none
    parallel_for(done, [&](long lo, long hi) {
        for (long jj = lo; jj < hi; ++jj) {
            const int i = split[jj], b = bslot[jj];
            const float *S = stats + (long)i * SAD_STAT_LD;
            const double mass = S[0], E = S[1];
            double ox = 0.0, oy = 0.0;
            bool have_axis = false;
            if (mass >= cfg->min_mass && E > 0.0) {
                const double mx = S[2] / E, my = S[3] / E;
                const double cxx = S[4] / E - mx * mx, cxy = S[5] / E - mx * my, cyy = S[6] / E - my * my;
                double lam, ex, ey;
                principal_axis(cxx, cxy, cyy, lam, ex, ey);
                if (std::isfinite(lam) && lam > 0.0) {
                    const double h = 0.5 * std::sqrt(lam);
                    ox = h * ex;
                    oy = h * ey;
                    have_axis = true;
                }
            }
            if (!have_axis) {
                const int c = img.col(P(PX, i)), r = img.row(P(PY, i));
                double gx = (img.lum(c + 1, r - 1) + 2.0 * img.lum(c + 1, r) + img.lum(c + 1, r + 1)) -
                            (img.lum(c - 1, r - 1) + 2.0 * img.lum(c - 1, r) + img.lum(c - 1, r + 1));
                double gy = (img.lum(c - 1, r + 1) + 2.0 * img.lum(c, r + 1) + img.lum(c + 1, r + 1)) -
                            (img.lum(c - 1, r - 1) + 2.0 * img.lum(c, r - 1) + img.lum(c + 1, r - 1));
                const double gn = std::sqrt(gx * gx + gy * gy);
                if (gn > 0.0) {
                    gx /= gn;
                    gy /= gn;
                } else {
                    gx = 1.0;
                    gy = 0.0;
                }
                const double h = 0.5 * std::sqrt(std::max(mass, 1.0) / M_PI);
                ox = h * gx;
                oy = h * gy;
            }
            const double px = P(PX, i), py = P(PY, i);
            const double cx[2] = {px - ox, px + ox}, cy[2] = {py - oy, py + oy};
            const int slot[2] = {i, b};
            float par[SAD_NPARAM];
            for (int q = 0; q < SAD_NPARAM; ++q)
                par[q] = P(q, i);
            for (int h = 0; h < 2; ++h) {
                const int s = slot[h];
                for (int q = 0; q < SAD_NPARAM; ++q) {
                    P(q, s) = par[q];
                    m[q * st + s] = v[q * st + s] = 0.0f;
                }
                const double x = std::min(std::max(cx[h], 0.0), (double)W);
                const double y = std::min(std::max(cy[h], 0.0), (double)H);
                P(PX, s) = (float)x;
                P(PY, s) = (float)y;
                P(PR, s) = par[PR] * cfg->shrink;
                P(PLT, s) = par[PLT] + lshrink;
                const float *tc = target + 3 * ((long)img.row(y) * W + img.col(x));
                P(PCR, s) = tc[0];
                P(PCG, s) = tc[1];
                P(PCB, s) = tc[2];
            }
            // seed child B into the list of its pixel's map entry and of the 4
            // neighbour entries (last place)
            const int bc = img.col(P(PX, b)) / cell, br = img.row(P(PY, b)) / cell;
            const int dc[5] = {0, -1, 1, 0, 0}, dr[5] = {0, 0, 0, -1, 1};
            for (int q = 0; q < 5; ++q) {
                const int c = bc + dc[q], r = br + dr[q];
                if (c >= 0 && c < Wm && r >= 0 && r < Hm)
                    seed_e[5 * jj + q] = (long)r * Wm + c;
            }
        }
    });
    // seeding, in split order; a list that already holds the ID keeps its last place
    for (long jj = 0; jj < done; ++jj) {
        const uint32_t b = (uint32_t)bslot[jj];
        for (int q = 0; q < 5; ++q) {
            const long e = seed_e[5 * jj + q];
            if (e < 0)
                continue;
            if (cand) {
                uint32_t *L = cand + e * SAD_K;
                if (std::find(L, L + SAD_K, b) == L + SAD_K)
                    L[SAD_K - 1] = b;
            }
            if (seeds) {
                seeds[2 * n_seeds] = (uint32_t)e;
                seeds[2 * n_seeds + 1] = b;
                ++n_seeds;
            }
        }
    }
    if (seeds && n_seeds > 1) {
        // grouped by entry, write order kept within an entry
        std::vector<std::pair<uint32_t, uint32_t>> pr((size_t)n_seeds);
        for (long q = 0; q < n_seeds; ++q)
            pr[q] = {seeds[2 * q], seeds[2 * q + 1]};
        std::stable_sort(pr.begin(), pr.end(),
                         [](const std::pair<uint32_t, uint32_t> &a, const std::pair<uint32_t, uint32_t> &b) {
                             return a.first < b.first;
                         });
        for (long q = 0; q < n_seeds; ++q) {
            seeds[2 * q] = pr[q].first;
            seeds[2 * q + 1] = pr[q].second;
        }
    }
    *n_slots = count;
    if (seeds)
        *n_seeds_out = n_seeds;
    if (n_split_out)
        *n_split_out = done;
    if (n_pruned_out)
        *n_pruned_out = pruned;
    return short_of_slots ? SAD_ERR_CAPACITY : SAD_OK;
}

extern "C" int sad_densify_prune(float *sites, float *m, float *v, float *removal, int *n_slots, int capacity,
                                 int stride, uint32_t *cand, int W, int H, const float *target,
                                 const sad_budget_cfg *cfg, uint64_t seed)
{
    (void)seed;  // reserved: no rule draws a random number
    if (!sites || !m || !v || !removal || !n_slots || !cand || !target || !cfg)
        return SAD_ERR_ARG;
    const int n = *n_slots;
    if (n < 0 || stride < 1 || n > stride || capacity < n || capacity > stride || W < 1 || H < 1 ||
        W > SAD_MAX_DIM || H > SAD_MAX_DIM)
        return SAD_ERR_ARG;
    if (!(cfg->split_frac >= 0.0f && cfg->split_frac <= 1.0f && cfg->prune_frac >= 0.0f &&
          cfg->prune_frac <= 1.0f && cfg->shrink > 0.0f && cfg->min_mass >= 0.0f))
        return SAD_ERR_ARG;
    std::vector<float> stats((size_t)stride * SAD_STAT_LD, 0.0f);
    host_stats(sites, n, stride, cand, W, H, target, stats.data());
    const int rc = sad_densify_prune_stats(sites, m, v, stride, capacity, n_slots, stats.data(), removal, cand, W, H, 1,
                                           target, cfg, nullptr, nullptr, nullptr, 0, nullptr);
    if (rc == SAD_OK || rc == SAD_ERR_CAPACITY)
        std::fill(removal, removal + *n_slots, 0.0f);
    return rc;
}
