// sad_kernels.hip -- gfx950 kernels and the C ABI of libsad (declared in include/sad.h).
//
// Soft Anisotropic Diagrams (SAD): top-K candidate maintenance (propagation with
// injection, the jump-flood prepass, the exact top-K; per pixel or on a
// downscaled grid), the temperature-softmax render, its analytic backward, Adam,
// budget-control statistics, the packed candidate-site buffer and the 16-byte
// evaluation format with random-access queries.  Formulas follow the
// woaixuexisr.github.io reading note ("Key designs" 1-4), the luckyiyi.github.io
// project page ("Method"), the paperlayer.ai summary (sections 4-5, Appendix B)
// and the 69574.cn article (section 5); each kernel names the passage it
// implements.
//
// Execution model: image-space kernels cover the image with 16x16-pixel tiles,
// one 256-thread workgroup (four wave64s) per tile, one pixel per lane (the fused
// backward: 512 threads, two lanes per pixel).  Tiles
// are handed out so that each XCD (workgroup IDs are dealt round-robin over the
// 8 XCDs) receives one contiguous band of tiles, which keeps the site gathers and
// neighbour-list re-reads of a band inside that XCD's L2.  Per-site kernels use
// 256 threads per workgroup, one slot per thread.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sad.h"

namespace {

constexpr int K = SAD_K;
constexpr uint32_t NONE = SAD_INVALID;
constexpr int TILE = 16;
constexpr int BLOCK = TILE * TILE;
constexpr int NXCD = 8;
constexpr int HASH_PROBES = 12;

// Site planes (order of the site buffer).
constexpr int PX = SAD_X, PY = SAD_Y, PLT = SAD_LOGTAU, PR = SAD_R, PCR = SAD_CR, PCG = SAD_CG, PCB = SAD_CB,
              PDX = SAD_DIRX, PDY = SAD_DIRY, PA = SAD_A;

// Workgroup ID -> logical tile so that the workgroups of one XCD cover a
// contiguous run of tiles (a bijection on [0, nb)).
__device__ __forceinline__ int xcd_band(int bid, int nb)
{
    const int q = nb / NXCD, rem = nb % NXCD;
    const int x = bid % NXCD, i = bid / NXCD;
    return x * q + min(x, rem) + i;
}

// The candidate map's grid (summary, Appendix B.3 "Candidate field"): cells of
// c x c pixels, Wm = ceil(W/c) of them per row; pixel (col, row) reads the list of
// cell (col/c, row/c), and a cell's candidates are selected at its centred UV,
// ((cx + 1/2) sx, (cy + 1/2) sy) px with sx = W/Wm, sy = H/Hm.  c = 1 is the
// per-pixel map (sx = sy = 1).
struct MapGrid {
    int c, Wm;
    float sx, sy;

    // list index of pixel (col, row), whose image index is p
    __device__ __forceinline__ long entry(long p, int col, int row) const
    {
        return c == 1 ? p : (long)(row / c) * Wm + col / c;
    }
};

__device__ __forceinline__ bool finitef(float v) { return __builtin_isfinite(v); }

// Hardware square root, reciprocal and reciprocal square root (1 ulp).  The
// scores, blends and updates here tolerate one ulp, while the correctly rounded
// sequences the compiler emits for sqrtf and '/' cost 10-18 instructions each
// and sit in the innermost loops.  Denormal inputs are not relied on: the
// arguments are squared distances (where 1e-38 px^2 is immaterial) or sums
// bounded below (see the call sites).
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// Metric frame of one site: u = dir/|dir| (u = (1,0) if |dir|^2 < 1e-30) and e^{+-a}.
struct Frame {
    float ux, uy, E, iE;
};

__device__ __forceinline__ Frame make_frame(float dx, float dy, float a)
{
    Frame f;
    const float n2 = dx * dx + dy * dy;
    f.ux = 1.0f;
    f.uy = 0.0f;
    if (n2 >= 1e-30f) {
        const float inv = hw_rsq(n2);  // n2 >= 1e-30
        f.ux = dx * inv;
        f.uy = dy * inv;
    }
    f.E = __expf(a);
    f.iE = __expf(-a);
    return f;
}

// d = s*||x - p||_G - s*r with ||delta||_G^2 = e^a (u.delta)^2 + e^-a (v.delta)^2,
// v = (-u_y, u_x)  (reading note, key design 1).
// (Multiply-adds are written as fmaf so that no contraction is left to the
// compiler: the forward rounds the same way in every kernel that inlines it.)
__device__ __forceinline__ float score_frame(const Frame &f, float px, float py, float r, float X, float Y, float s)
{
    const float ex = X - px, ey = Y - py;
    const float al = fmaf(f.ux, ex, f.uy * ey);
    const float be = fmaf(f.ux, ey, -(f.uy * ex));
    const float q = hw_sqrt(fmaf(f.E * al, al, f.iE * be * be));
    return fmaf(s, q, -(s * r));
}

// ---------------------------------------------------------------------------
// Site record, 64 bytes per site, derived from the ten parameters: everything an
// image-space kernel needs about a site in one contiguous, 16-byte-aligned block,
// so a random access costs a few vector loads instead of one gather per
// parameter plane.  The first 32 bytes are the scoring record the candidate
// search reads -- the fp32 counterpart of the pages' compact candidate-site
// buffer (summary, Appendix B.2 "Packed candidate sites"):
//   [0]  x   y   r   Ux     [1]  Uy  Vx  Vy  tau
//   [2]  R   G   B   1/|dir|  [3]  ux  uy  E   1/E
// with u = dir/|dir| (u = (1,0) when |dir|^2 < 1e-30), E = e^a, tau = e^{log tau},
// U = e^{a/2} u and V = e^{-a/2} u, so ||delta||_G^2 = (U.delta)^2 + (V x delta)^2
// = e^a alpha^2 + e^-a beta^2 -- a sum of squares, as in the definition (reading
// note, key design 1).  1/|dir| is 0 for a degenerate direction.
constexpr int RLD4 = SAD_REC_LD / 4;  // float4 per record

// record of a site whose ten parameters are in registers
__device__ __forceinline__ void make_record_v(const float (&p)[SAD_NPARAM], float4 (&o)[RLD4])
{
    const float x = p[PX], y = p[PY], lt = p[PLT], r = p[PR];
    const float c0 = p[PCR], c1 = p[PCG], c2 = p[PCB];
    const float dx = p[PDX], dy = p[PDY], a = p[PA];
    const Frame f = make_frame(dx, dy, a);
    const float sE = __expf(0.5f * a), siE = __expf(-0.5f * a);
    const float n2 = dx * dx + dy * dy;
    o[0] = make_float4(x, y, r, sE * f.ux);
    o[1] = make_float4(sE * f.uy, siE * f.ux, siE * f.uy, __expf(lt));
    o[2] = make_float4(c0, c1, c2, n2 >= 1e-30f ? hw_rsq(n2) : 0.0f);
    o[3] = make_float4(f.ux, f.uy, f.E, f.iE);
}

__device__ __forceinline__ void make_record(const float *__restrict__ S, long st, int i, float4 (&o)[RLD4])
{
    float p[SAD_NPARAM];
#pragma unroll
    for (int k = 0; k < SAD_NPARAM; ++k)
        p[k] = S[k * st + i];
    make_record_v(p, o);
}

__device__ __forceinline__ float geom_score(const float4 &g0, const float4 &g1, float X, float Y, float s)
{
    const float ex = X - g0.x, ey = Y - g0.y;
    const float t1 = g0.w * ex + g1.x * ey;  // e^{a/2} (u . delta)
    const float t2 = g1.y * ey - g1.z * ex;  // e^{-a/2} (u x delta)
    const float q = hw_sqrt(t1 * t1 + t2 * t2);
    return s * q - s * g0.z;
}

// Selection site formats: the candidate kernels score either from the 64-byte
// records (their first 32 bytes) or from the 16-byte packed candidate-site buffer
// of float16 pairs (summary, Appendix B.2 "Packed candidate sites"): words
// (x, y), (log tau, r), (dir_x, dir_y), (a, 0), first field in the low half.  Both
// yield the same scoring record (x, y, r, Ux | Uy, Vx, Vy, -); decoding the packed
// words costs a few VALU per fetch and halves the bytes fetched per candidate.
// A third source, the site planes themselves (float [10][stride]), serves the
// entry points that take the site buffer directly: the scoring record is then
// derived per fetch with the same operations make_record_v performs, so every
// score is bit-identical to the one computed from a fresh record.
constexpr int SEL_REC = SAD_SEL_REC64, SEL_PACKED = SAD_SEL_PACKED16, SEL_SOA = 2;

// Where a kernel reads sites: the records or packed words (G), or the planes
// (S with plane stride st).
struct SiteSrc {
    const float4 *G;
    const float *S;
    long st;
};

__device__ __forceinline__ float half_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16)); }

// Scoring record of site `id`: the first 32 bytes of its record, its packed words
// decoded, or the same 32 bytes derived from the planes.
template <int FMT>
__device__ __forceinline__ void load_sel(const SiteSrc &src, uint32_t id, float4 &g0, float4 &g1)
{
    if constexpr (FMT == SEL_REC) {
        g0 = src.G[RLD4 * (size_t)id];
        g1 = src.G[RLD4 * (size_t)id + 1];
    } else if constexpr (FMT == SEL_SOA) {
        const float *S = src.S + id;
        const long st = src.st;
        const float x = S[PX * st], y = S[PY * st], r = S[PR * st], dx = S[PDX * st], dy = S[PDY * st],
                    a = S[PA * st];
        const Frame f = make_frame(dx, dy, a);
        const float sE = __expf(0.5f * a), siE = __expf(-0.5f * a);
        g0 = make_float4(x, y, r, sE * f.ux);
        g1 = make_float4(sE * f.uy, siE * f.ux, siE * f.uy, 0.0f);
    } else {
        const float4 v = src.G[id];
        const uint32_t w0 = __float_as_uint(v.x), w1 = __float_as_uint(v.y), w2 = __float_as_uint(v.z),
                       w3 = __float_as_uint(v.w);
        const float dx = half_lo(w2), dy = half_hi(w2), a = half_lo(w3);
        const float n2 = dx * dx + dy * dy;
        float ux = 1.0f, uy = 0.0f;
        if (n2 >= 1e-30f) {
            const float inv = hw_rsq(n2);
            ux = dx * inv;
            uy = dy * inv;
        }
        const float sE = __expf(0.5f * a), siE = __expf(-0.5f * a);
        g0 = make_float4(half_lo(w0), half_hi(w0), half_hi(w1), sE * ux);
        g1 = make_float4(sE * uy, siE * ux, siE * uy, 0.0f);
    }
}

template <int FMT>
__device__ __forceinline__ float geom_score_id(const SiteSrc &src, uint32_t id, float X, float Y, float s,
                                               bool &usable)
{
    float4 g0, g1;
    load_sel<FMT>(src, id, g0, g1);
    usable = !(g0.x < 0.0f);
    return geom_score(g0, g1, X, Y, s);
}

__global__ __launch_bounds__(256) void k_site_records(const float *__restrict__ S, int n_slots, int stride,
                                                      float4 *__restrict__ G)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n_slots)
        return;
    float4 o[RLD4];
    make_record(S, stride, i, o);
#pragma unroll
    for (int j = 0; j < RLD4; ++j)
        G[RLD4 * (size_t)i + j] = o[j];
}

// Packed candidate-site words of slot i (binary16, round to nearest even, as the
// conversion instruction does by default); an inactive slot (x < 0) packs x = -1.
__device__ __forceinline__ uint32_t f16_bits(float v) { return __builtin_bit_cast(unsigned short, (_Float16)v); }

__device__ __forceinline__ uint4 pack_site_v(const float (&p)[SAD_NPARAM])
{
    const uint32_t hx = p[PX] < 0.0f ? 0xBC00u : f16_bits(p[PX]);
    return make_uint4(hx | (f16_bits(p[PY]) << 16), f16_bits(p[PLT]) | (f16_bits(p[PR]) << 16),
                      f16_bits(p[PDX]) | (f16_bits(p[PDY]) << 16), f16_bits(p[PA]));
}

__device__ __forceinline__ uint4 pack_site(const float *__restrict__ S, long st, int i)
{
    float p[SAD_NPARAM];
#pragma unroll
    for (int k = 0; k < SAD_NPARAM; ++k)
        p[k] = S[k * st + i];
    return pack_site_v(p);
}

__global__ __launch_bounds__(256) void k_pack_sites(const float *__restrict__ S, int n_slots, int stride,
                                                    uint4 *__restrict__ P)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n_slots)
        P[i] = pack_site(S, stride, i);
}

// A selected list is written once and read by the next pass: stored as a
// stream (non-temporal), so a pass's 32 bytes per entry of output do not evict
// the site records and screen words that its gathers reuse from L2.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_list(uint4 *__restrict__ out, long p, const uint64_t (&k)[SAD_K])
{
    u32x4 *o = reinterpret_cast<u32x4 *>(out) + 2 * p;
    __builtin_nontemporal_store(u32x4{(uint32_t)k[0], (uint32_t)k[1], (uint32_t)k[2], (uint32_t)k[3]}, o);
    __builtin_nontemporal_store(u32x4{(uint32_t)k[4], (uint32_t)k[5], (uint32_t)k[6], (uint32_t)k[7]}, o + 1);
}

// ---------------------------------------------------------------------------
// Counter-based injection (paperlayer.ai summary, Appendix B.3: the pass word and
// the pixel ID seed xorshift).  pcg hash: Jarzynski & Olano, JCGT 2020;
// xorshift32 (13,17,5): Marsaglia 2003; range: Lemire's multiply-shift.
__device__ __forceinline__ uint32_t pcg_hash(uint32_t v)
{
    const uint32_t state = v * 747796405u + 2891336453u;
    const uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
    return (word >> 22u) ^ word;
}

__device__ __forceinline__ uint32_t xorshift32(uint32_t x)
{
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
}

// ---------------------------------------------------------------------------
// Lane moves without the LDS: a DPP move of x (CTRL: the DPP control word; ROWS:
// the rows written, others keep 0), and an inclusive prefix sum over a wave.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes (lanes whose DPP source lies outside
// the row add 0): within each 16-lane row by row_shr 1, 2, 4, 8, then the last
// lane of row 0 and of row 2 into rows 1 and 3 (row_bcast:15), then lane 31 into
// rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    x += dpp_u<0x111, 0xF>(x);
    x += dpp_u<0x112, 0xF>(x);
    x += dpp_u<0x114, 0xF>(x);
    x += dpp_u<0x118, 0xF>(x);
    x += dpp_u<0x142, 0xA>(x);
    x += dpp_u<0x143, 0xC>(x);
    return x;
}

// ---------------------------------------------------------------------------
// Inserts one list's IDs into an LDS hash table of TB slots keyed by site ID
// (multiplicative hash, CAS insert -- summary, B.4; double hashing with an odd
// step, <= HASH_PROBES probes: at the ~30 % load of a converged map's tile no ID
// then fails to find a slot, whereas linear probing's clusters made a few tiles
// per launch take the slow spill path and finish last).  refs[k]: the slot,
// REF_SPILL | ID if every probe is taken by other IDs,
// REF_NONE when ids[k] >= n_slots.  (Measured on gfx950: one CAS per probe, ID
// by ID, beats reading the slot first and beats issuing the CAS of all IDs of a
// list at once -- same-address atomics from many lanes serialise.)
constexpr uint32_t REF_NONE = 0xFFFFFFFFu;
constexpr uint32_t REF_SPILL = 0x80000000u;  // | site ID

template <int TB, int N, bool COUNT = false>
__device__ __forceinline__ void table_insert_ids(uint32_t *key, const uint32_t (&ids)[N], uint32_t n_slots,
                                                 uint32_t (&refs)[N], uint32_t *n_new = nullptr)
{
    constexpr int SHIFT = TB == 256 ? 24 : TB == 512 ? 23 : 21;
    static_assert(TB == 256 || TB == 512 || TB == 2048, "table size");
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const uint32_t c = ids[k];
        uint32_t r = REF_NONE;
        if (c < n_slots) {
            r = REF_SPILL | c;
            const uint32_t h0 = (c * 2654435761u) >> SHIFT;
            const uint32_t step = ((c * 0x85EBCA6Bu) >> SHIFT) | 1u;
            for (int pr = 0; pr < HASH_PROBES; ++pr) {
                const uint32_t sl = (h0 + (uint32_t)pr * step) & (TB - 1);
                const uint32_t prev = atomicCAS(&key[sl], NONE, c);
                if (prev == NONE || prev == c) {
                    if (COUNT && prev == NONE)
                        atomicAdd(n_new, 1u);  // distinct IDs of the lists inserted
                    r = sl;
                    break;
                }
            }
        }
        refs[k] = r;
    }
}

// ---------------------------------------------------------------------------
// Propagation pass (reading note, key design 3; summary, section 4 and B.3).
//
// One 16x16 tile per workgroup, one pixel per lane.  A pixel's candidates are
// its own list, the lists at +-jump in x and y (skipped outside the image) and
// n_inject injected IDs.  The lists the tile needs -- its own block plus four
// strips of width min(jump, 16) beyond its edges -- are loaded once; every ID in
// them goes into an LDS site table (hash keyed by ID, CAS insert) and
// each list entry is replaced by its table slot.  Each distinct site is then
// gathered once per tile and its metric frame computed once, so scoring a list
// candidate costs two LDS reads instead of six scattered global loads.  IDs the
// table cannot hold ("spills") and injected IDs are read from global memory.
//
// Selection: candidates are ranked by a 64-bit key (order-preserving bits of d,
// then the ID) -- the (d, ID) order.  A candidate is inserted when its key beats
// the current K-th and its ID is not yet held; a repeat of an ID that was
// rejected or evicted earlier is rejected again (the K-th key only decreases),
// so the result is the top-K of the deduplicated union.
__device__ __forceinline__ uint64_t rank_key(float d, uint32_t id)
{
    uint32_t u = __float_as_uint(d + 0.0f);  // -0 -> +0
    u ^= (u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;
    return ((uint64_t)u << 32) | id;
}

__device__ __forceinline__ void cswap(uint64_t &a, uint64_t &b)
{
    const bool lt = b < a;
    const uint64_t lo = lt ? b : a, hi = lt ? a : b;
    a = lo;
    b = hi;
}

struct TopK64 {
    uint64_t k[K];

    // Sorts 8 keys with Batcher's odd-even merge network (19 comparators).
    __device__ __forceinline__ void set_sorted(uint64_t (&v)[K])
    {
        cswap(v[0], v[1]); cswap(v[2], v[3]); cswap(v[4], v[5]); cswap(v[6], v[7]);
        cswap(v[0], v[2]); cswap(v[1], v[3]); cswap(v[4], v[6]); cswap(v[5], v[7]);
        cswap(v[1], v[2]); cswap(v[5], v[6]); cswap(v[0], v[4]); cswap(v[3], v[7]);
        cswap(v[1], v[5]); cswap(v[2], v[6]); cswap(v[1], v[4]); cswap(v[3], v[6]);
        cswap(v[2], v[4]); cswap(v[3], v[5]); cswap(v[3], v[4]);
#pragma unroll
        for (int j = 0; j < K; ++j)
            k[j] = v[j];
    }
    __device__ __forceinline__ bool holds(uint32_t id) const
    {
        bool hit = false;
#pragma unroll
        for (int j = 0; j < K; ++j)
            hit |= ((uint32_t)k[j] == id);
        return hit;
    }
    // Precondition: key < k[K-1] and the key's ID is not held.
    __device__ __forceinline__ void insert(uint64_t key)
    {
#pragma unroll
        for (int j = K - 1; j > 0; --j)
            k[j] = (key < k[j - 1]) ? k[j - 1] : ((key < k[j]) ? key : k[j]);
        k[0] = (key < k[0]) ? key : k[0];
    }
    // A candidate known not to be held.
    __device__ __forceinline__ void consider_new(uint32_t id, float d, bool usable)
    {
        if (!usable || !finitef(d))
            return;
        const uint64_t key = rank_key(d, id);
        if (key < k[K - 1])
            insert(key);
    }
    // A candidate that may already be held.
    __device__ __forceinline__ void consider(uint32_t id, float d, bool usable)
    {
        if (!usable || !finitef(d))
            return;
        const uint64_t key = rank_key(d, id);
        if (key < k[K - 1] && !holds(id))
            insert(key);
    }
};

// ---------------------------------------------------------------------------
// Candidate screen.  Most candidates a selection pass offers cannot enter the
// list: the injected IDs are uniform over the whole image, and at large jumps the
// neighbour lists name sites about `jump` pixels away.  Fetching their 32-byte
// scoring records is what those passes spend their time on (the records of a
// 2k or 4k fit do not stay in L2), so each site also has a 4-byte screen word
// from which a lane can prove, before any record fetch, that a candidate's score
// exceeds the list's current K-th score.  With A = e^{|a|/2} the metric obeys
// ||delta||_G >= ||delta|| / A, hence d = s(||delta||_G - r) > kth whenever
//   ||delta|| > A (max(kth, 0)/s + max(r, 0)),
// and the word holds enough to bound both sides:
//   bits 0..11   qx = floor(x * 4096 / W), bits 12..23  qy = floor(y * 4096 / H):
//                the site lies in cell qx of width W/4096 (qy likewise), so the
//                distance from the scoring point to that cell bounds ||delta||
//   bits 24..27  ca: A_hat = 2^(ca/2) >= A
//   bits 28..31  cr: R_hat = 2^(cr - 8) >= A_hat max(r, 0), 0 for cr = 0
// ca = 15 or cr = 15 mark a site the word cannot bound (inactive, non-finite,
// outside the image, |a| > 9.7 or A_hat r > 64 px): it is never screened out.
// The test adds a relative slack of 2^-10 and an absolute one of 1/64 px +
// 2^-16 R_hat, far above the float32 rounding of the cell bounds and of the score,
// so a screened-out candidate is one the full test would have rejected: the
// selected lists are the same bits with or without the screen.
constexpr float SCR_Q = 4096.0f;

__device__ __forceinline__ uint32_t screen_word(float x, float y, float r, float a, float qsx, float qsy)
{
    constexpr uint32_t NO_BOUND = 15u << 24;
    const float fx = x * qsx, fy = y * qsy;
    if (!(x >= 0.0f && y >= 0.0f && fx < SCR_Q + 0.5f && fy < SCR_Q + 0.5f) || !finitef(r) || !finitef(a))
        return NO_BOUND;
    const float fca = ceilf(fabsf(a) * 1.44269504f + 0.01f);  // |a| / ln 2, rounded up with slack
    if (!(fca <= 14.0f))
        return NO_BOUND;
    const int ca = (int)fca;
    const float Ahat = ldexpf((ca & 1) ? 1.41421366f : 1.0f, ca >> 1);  // 1.41421366 > sqrt(2)
    const float rr = fmaxf(r, 0.0f) * Ahat;
    uint32_t cr = 0;
    if (rr > 0.0f) {
        const float e = ceilf(__log2f(rr) + 0.01f) + 8.0f;
        if (!(e <= 14.0f))
            return NO_BOUND;
        cr = (uint32_t)fmaxf(e, 1.0f);
    }
    const uint32_t qx = (uint32_t)fminf(floorf(fx), SCR_Q - 1.0f), qy = (uint32_t)fminf(floorf(fy), SCR_Q - 1.0f);
    return qx | (qy << 12) | ((uint32_t)ca << 24) | (cr << 28);
}

// The screen of a selection kernel: the words (NULL: no screening) and the cell
// size W/4096, H/4096 in pixels.
struct Screen {
    const uint32_t *w;
    float cw, ch, inv_s;  // inv_s = max(W, H)
};

// Score of a ranking key (the inverse of rank_key's order-preserving map).
__device__ __forceinline__ float key_score(uint64_t key)
{
    uint32_t u = (uint32_t)(key >> 32);
    u ^= (u & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu;
    return __uint_as_float(u);
}

// True when site id scored at (X, Y) provably ranks after `kth` (the key of the
// list's K-th entry; ~0 while the list has a free place).
__device__ __forceinline__ bool screened_out_word(const Screen &sc, uint32_t v, float X, float Y, uint64_t kth)
{
    if (kth == ~0ull)
        return false;
    const uint32_t ca = (v >> 24) & 15u, cr = v >> 28;
    if (ca == 15u || cr == 15u)
        return false;
    const float Ahat = ldexpf((ca & 1u) ? 1.41421366f : 1.0f, (int)(ca >> 1));
    const float Rhat = cr ? ldexpf(1.0f, (int)cr - 8) : 0.0f;
    const float x0 = (float)(v & 0xFFFu) * sc.cw, y0 = (float)((v >> 12) & 0xFFFu) * sc.ch;
    const float dx = fmaxf(fmaxf(x0 - X, X - (x0 + sc.cw)), 0.0f);
    const float dy = fmaxf(fmaxf(y0 - Y, Y - (y0 + sc.ch)), 0.0f);
    const float kd = fmaxf(key_score(kth), 0.0f) * sc.inv_s;
    const float B = fmaf(Ahat * kd, 1.0009766f, Rhat) + fmaf(Rhat, 1.5258789e-5f, 0.015625f);
    return dx * dx + dy * dy > B * B;
}

__device__ __forceinline__ bool screened_out(const Screen &sc, uint32_t id, float X, float Y, uint64_t kth)
{
    return sc.w && kth != ~0ull && screened_out_word(sc, sc.w[id], X, Y, kth);
}

// Offers the n_inject injected IDs of map entry `pix` to its list (summary, B.3;
// the draw is described at sad_topk_propagate), each screened before its record
// is fetched.  (Loading the screen words of the first eight when the pass starts,
// to hide their latency, was measured slower: 191 -> 199 us for a 2048x2048 map.)
template <int FMT>
__device__ __forceinline__ void inject(const SiteSrc &src, const Screen &sc, uint32_t seed_h, uint32_t pix,
                                       uint32_t n_slots, int n_inject, float X, float Y, float s, TopK64 &best)
{
    const uint32_t h = pcg_hash(seed_h ^ pix);
    uint32_t x = h ? h : 0x9E3779B9u;
    for (int j = 0; j < n_inject; ++j) {
        x = xorshift32(x);
        const uint32_t c = (uint32_t)(((uint64_t)x * (uint64_t)n_slots) >> 32);
        if (c < n_slots && !screened_out(sc, c, X, Y, best.k[K - 1])) {
            bool usable;
            const float d = geom_score_id<FMT>(src, c, X, Y, s, usable);
            best.consider(c, d, usable);
        }
    }
}

// Screen words of slots [0, n_slots) (see screen_word; qsx = 4096/W, qsy = 4096/H).
__global__ __launch_bounds__(256) void k_site_screen(const float *__restrict__ S, int n_slots, int stride, float qsx,
                                                     float qsy, uint32_t *__restrict__ scr)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n_slots)
        return;
    const long st = stride;
    scr[i] = screen_word(S[PX * st + i], S[PY * st + i], S[PR * st + i], S[PA * st + i], qsx, qsy);
}

template <int KK, int TB>
struct PropShared {
    // The hash keys are needed until the records are loaded; from then on a
    // slot's ID travels in the last float of its record (the scoring record's
    // tau, which scoring does not use).
    // Records and lists are split into 16-byte halves kept in separate arrays, so
    // lanes reading consecutive lists (or slots) read consecutive 16-byte words.
    union {
        uint32_t key[TB];
        float4 rec0[TB];                        // scoring record, bytes 0..15
    } t;
    float4 rec1[TB];                            // scoring record, bytes 16..31
    uint4 ref[BLOCK + 4 * TILE * KK];           // per region list: 8 x 16-bit refs (REF16_*)
    uint32_t seen[TB / 32][BLOCK];              // per pixel: slots already taken (word-major)
};

// A list entry's table reference in 16 bits: the slot, or REF16_SPILL (the ID
// found no slot: it is read again from the list in global memory), or
// REF16_NONE (no site).  Half the LDS of 32-bit refs: 21 KB per workgroup, so
// seven workgroups fit a CU instead of six.
constexpr uint32_t REF16_NONE = 0xFFFFu, REF16_SPILL = 0xFFFEu;

template <int TB>
__device__ __forceinline__ uint32_t ref16(uint32_t ref)
{
    return ref < (uint32_t)TB ? ref : ref == REF_NONE ? REF16_NONE : REF16_SPILL;
}

template <int TB>
__device__ __forceinline__ uint4 pack_refs16(const uint32_t (&r)[K])
{
    return make_uint4(ref16<TB>(r[0]) | ref16<TB>(r[1]) << 16, ref16<TB>(r[2]) | ref16<TB>(r[3]) << 16,
                      ref16<TB>(r[4]) | ref16<TB>(r[5]) << 16, ref16<TB>(r[6]) | ref16<TB>(r[7]) << 16);
}

// Absolute pixel of region list r: the own block, then the left, right, top and
// bottom strips, each KK lists across by 16 along the tile edge (only the first
// min(jump, 16) across are used).
__device__ __forceinline__ void region_pixel(int r, int c0, int r0, int jump, int strip_len, int &col, int &row,
                                             int &across)
{
    if (r < BLOCK) {
        col = c0 + (r & (TILE - 1));
        row = r0 + r / TILE;
        across = 0;
        return;
    }
    const int q = r - BLOCK;
    const int sidx = q / strip_len, w = q - sidx * strip_len;
    const int i = w / TILE, j = w - i * TILE;
    const int far = max(TILE, jump);
    across = i;
    switch (sidx) {
    case 0: col = c0 - jump + i; row = r0 + j; break;
    case 1: col = c0 + far + i; row = r0 + j; break;
    case 2: col = c0 + j; row = r0 - jump + i; break;
    default: col = c0 + j; row = r0 + far + i; break;
    }
}

template <int KK, int TB, int FMT>
__global__ __launch_bounds__(BLOCK) void k_propagate(SiteSrc src, Screen sc, uint32_t n_slots,
                                                     const uint4 *__restrict__ cin, uint4 *__restrict__ cout, int W,
                                                     int H, int jump, uint32_t seed_h, int n_inject, float s, float sx,
                                                     float sy, int tiles_x, int nb)
{
    __shared__ PropShared<KK, TB> L;
    const int tid = threadIdx.x;
    const int t = xcd_band(blockIdx.x, nb);
    const int c0 = (t % tiles_x) * TILE, r0 = (t / tiles_x) * TILE;
    const int lc = tid & (TILE - 1), lr = tid / TILE;
    const int col = c0 + lc, row = r0 + lr;
    const int kk = min(jump, TILE);
    const int strip_len = TILE * KK;
    const int nlists = BLOCK + 4 * strip_len;
    // Region list r is loaded with its two 16-byte halves swapped when r is odd
    // (the quarter-list loads of the jump-1 strips excepted), so that
    // neighbouring lanes insert different list places in one CAS instruction:
    // CAS lanes that name one LDS address serialise.  Refs follow the loaded
    // order; only a spill's re-read from global memory undoes the swap.  (Place
    // e holding entry e ^ (r & 7), with 8-byte loads and pair selects, measured
    // slower: 163 -> 169 us at 2048x2048, 131k sites.)
    auto list_swap = [&](int r) { return (KK == 1 && r >= BLOCK) ? 0 : (r & 1); };

    for (int sl = tid; sl < TB; sl += BLOCK)
        L.t.key[sl] = NONE;
#pragma unroll
    for (int w = 0; w < TB / 32; ++w)
        L.seen[w][tid] = 0u;
    __syncthreads();

    // phase 1: region lists -> table slots
    if constexpr (KK == 1) {
        // jump 1: every thread takes its pixel's list and two IDs of one of the 64
        // strip lists (a quarter list), both loads issued before the inserts, so no
        // thread inserts more than 10 IDs
        uint4 a = make_uint4(NONE, NONE, NONE, NONE), b = a;
        if (col < W && row < H) {
            const long p = (long)row * W + col;
            a = cin[2 * p + list_swap(tid)];
            b = cin[2 * p + 1 - list_swap(tid)];
        }
        const int sr = BLOCK + (tid >> 2), qq = tid & 3;
        int pc, pr, across;
        region_pixel(sr, c0, r0, jump, strip_len, pc, pr, across);
        uint2 q2 = make_uint2(NONE, NONE);
        if (pc >= 0 && pc < W && pr >= 0 && pr < H)
            q2 = reinterpret_cast<const uint2 *>(cin)[4 * ((long)pr * W + pc) + qq];
        const uint32_t ids[K] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t refs[K];
        table_insert_ids<TB>(L.t.key, ids, n_slots, refs);
        const uint32_t sids[2] = {q2.x, q2.y};
        uint32_t srefs[2];
        table_insert_ids<TB>(L.t.key, sids, n_slots, srefs);
        L.ref[tid] = pack_refs16<TB>(refs);
        reinterpret_cast<uint32_t *>(&L.ref[sr])[qq] = ref16<TB>(srefs[0]) | ref16<TB>(srefs[1]) << 16;
    } else {
        for (int r = tid; r < nlists; r += BLOCK) {
            int pc, pr, across;
            region_pixel(r, c0, r0, jump, strip_len, pc, pr, across);
            uint4 a = make_uint4(NONE, NONE, NONE, NONE), b = a;
            if (across < kk && pc >= 0 && pc < W && pr >= 0 && pr < H) {
                const long p = (long)pr * W + pc;
                a = cin[2 * p + list_swap(r)];
                b = cin[2 * p + 1 - list_swap(r)];
            }
            const uint32_t ids[K] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t refs[K];
            table_insert_ids<TB>(L.t.key, ids, n_slots, refs);
            L.ref[r] = pack_refs16<TB>(refs);
        }
    }
    __syncthreads();

    // phase 2: one scoring record per occupied slot (written over the keys)
    static_assert(TB == BLOCK, "one slot per lane");
    {
        const uint32_t c = L.t.key[tid];
        float4 g0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), g1 = g0;
        if (c != NONE)
            load_sel<FMT>(src, c, g0, g1);
        g1.w = __uint_as_float(c);
        __syncthreads();
        if (c != NONE) {
            L.t.rec0[tid] = g0;
            L.rec1[tid] = g1;
        }
    }
    __syncthreads();

    if (col >= W || row >= H)
        return;
    const float X = ((float)col + 0.5f) * sx, Y = ((float)row + 0.5f) * sy;
    auto rec_score_slot = [&](uint32_t sl, bool &usable, uint32_t &id) {
        const float4 g0 = L.t.rec0[sl], g1 = L.rec1[sl];
        usable = !(g0.x < 0.0f);
        id = __float_as_uint(g1.w);
        return geom_score(g0, g1, X, Y, s);
    };
    // marks slot sl as taken by this pixel; true if it was not taken before
    auto take = [&](uint32_t sl) {
        const uint32_t bit = 1u << (sl & 31u);
        return (atomicOr(&L.seen[sl >> 5][tid], bit) & bit) == 0u;
    };

    // the ID behind place e of region list r's refs, the list of pixel (pc, pr),
    // read again from global memory (spills)
    auto list_id = [&](int r, int pc, int pr, int e) {
        return reinterpret_cast<const uint32_t *>(cin)[(size_t)K * ((size_t)pr * W + pc) + (e ^ 4 * list_swap(r))];
    };
    TopK64 best;
    // own list: score its (deduplicated) table entries and sort them with a network
    const uint4 o16 = L.ref[tid];
    const uint32_t orefs[K] = {o16.x & 0xFFFFu, o16.x >> 16, o16.y & 0xFFFFu, o16.y >> 16,
                               o16.z & 0xFFFFu, o16.z >> 16, o16.w & 0xFFFFu, o16.w >> 16};
    {
        uint64_t v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t ref = orefs[k];
            v[k] = ~0ull;
            if (ref < (uint32_t)TB && take(ref)) {
                bool usable;
                uint32_t id;
                const float d = rec_score_slot(ref, usable, id);
                if (usable && finitef(d))
                    v[k] = rank_key(d, id);
            }
        }
        best.set_sorted(v);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (orefs[k] == REF16_SPILL) {
            const uint32_t c = list_id(tid, col, row, k);
            bool usable;
            const float d = geom_score_id<FMT>(src, c, X, Y, s, usable);
            best.consider(c, d, usable);
        }
    }
    // the four neighbour lists: only entries this pixel has not seen yet
    const int far = max(TILE, jump);
    const int r_l = col - jump >= 0 ? (lc - jump >= 0 ? lr * TILE + lc - jump : BLOCK + lc * TILE + lr) : -1;
    const int r_r = col + jump < W
                        ? (lc + jump < TILE ? lr * TILE + lc + jump : BLOCK + strip_len + (lc + jump - far) * TILE + lr)
                        : -1;
    const int r_t = row - jump >= 0 ? (lr - jump >= 0 ? (lr - jump) * TILE + lc : BLOCK + 2 * strip_len + lr * TILE + lc)
                                    : -1;
    const int r_b = row + jump < H ? (lr + jump < TILE ? (lr + jump) * TILE + lc
                                                       : BLOCK + 3 * strip_len + (lr + jump - far) * TILE + lc)
                                   : -1;
    // Entries new to this pixel, as one mask over the four lists (bit 8 li + k),
    // then scored in a single loop: the wave runs as many iterations as its
    // busiest lane has new entries in total, and each reads its ref from LDS.
    uint32_t fresh = 0;
#pragma unroll
    for (int li = 0; li < 4; ++li) {
        const int r = li == 0 ? r_l : li == 1 ? r_r : li == 2 ? r_t : r_b;
        if (r < 0)
            continue;
        const uint4 a = L.ref[r];
        const uint32_t refs[K] = {a.x & 0xFFFFu, a.x >> 16, a.y & 0xFFFFu, a.y >> 16,
                                  a.z & 0xFFFFu, a.z >> 16, a.w & 0xFFFFu, a.w >> 16};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t ref = refs[k];
            const bool f = ref < (uint32_t)TB ? take(ref) : ref != REF16_NONE;
            fresh |= f ? (1u << (li * K + k)) : 0u;
        }
    }
    while (fresh) {
        const int j = __builtin_ctz(fresh);
        fresh &= fresh - 1u;
        const int li = j / K;
        const int r = li == 0 ? r_l : li == 1 ? r_r : li == 2 ? r_t : r_b;
        const int e = j % K;
        const uint32_t ref = reinterpret_cast<const uint16_t *>(&L.ref[r])[e];
        bool usable;
        if (ref < (uint32_t)TB) {
            uint32_t id;
            const float d = rec_score_slot(ref, usable, id);
            best.consider_new(id, d, usable);
        } else {
            // a spilled entry: its ID from the neighbour's list in global memory
            const uint32_t c = list_id(r, li == 0 ? col - jump : li == 1 ? col + jump : col,
                                       li == 2 ? row - jump : li == 3 ? row + jump : row, e);
            if (!screened_out(sc, c, X, Y, best.k[K - 1])) {
                const float d = geom_score_id<FMT>(src, c, X, Y, s, usable);
                best.consider(c, d, usable);
            }
        }
    }
    // injected IDs (summary, B.3), screened before their records are fetched
    inject<FMT>(src, sc, seed_h, (uint32_t)row * (uint32_t)W + (uint32_t)col, n_slots, n_inject, X, Y, s, best);
    const long p = (long)row * W + col;
    store_list(cout, p, best.k);
}

// Propagation pass without a tile table, for the downscaled candidate grid (a
// tile of cells names more sites than a table holds): every candidate is scored
// from its site record (two 16-byte loads) and goes through the same (d, ID)
// selection with a duplicate check.  TW x TW map entries per workgroup: 16 for
// maps large enough to fill the chip with 16x16 tiles, 8 for small maps, which
// would otherwise leave most CUs idle.
template <int TW, int FMT>
__global__ __launch_bounds__(TW *TW) void k_propagate_direct(SiteSrc src, Screen sc, uint32_t n_slots,
                                                             const uint4 *__restrict__ cin, uint4 *__restrict__ cout,
                                                             int W, int H, int jump, uint32_t seed_h, int n_inject,
                                                             float s, float sx, float sy, int tiles_x, int nb)
{
    const int t = xcd_band(blockIdx.x, nb);
    const int col = (t % tiles_x) * TW + (threadIdx.x & (TW - 1));
    const int row = (t / tiles_x) * TW + (threadIdx.x / TW);
    if (col >= W || row >= H)
        return;
    const float X = ((float)col + 0.5f) * sx, Y = ((float)row + 0.5f) * sy;
    TopK64 best;
#pragma unroll
    for (int j = 0; j < K; ++j)
        best.k[j] = ~0ull;
    for (int li = 0; li < 5; ++li) {
        const int c = li == 1 ? col - jump : li == 2 ? col + jump : col;
        const int r = li == 3 ? row - jump : li == 4 ? row + jump : row;
        if (c < 0 || c >= W || r < 0 || r >= H)
            continue;
        const long q = (long)r * W + c;
        const uint4 a = cin[2 * q], b = cin[2 * q + 1];
        const uint32_t ids[K] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        // The records of the list's IDs not already held are fetched together,
        // then offered in order: one memory round trip per list rather than one
        // per candidate (the selection needs each score before the next offer,
        // the fetches do not).  Lists of nearby pixels share most of their sites,
        // so held IDs are skipped before the fetch (screening candidates first was
        // measured slower, 16.9 vs 14.1 ms for a 12-pass refresh of a 4096x4096 map without
        // injection); an ID a list repeats is caught by consider().
        float4 g0[K], g1[K];
        uint32_t need = 0u;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const bool nd = ids[k] < n_slots && !best.holds(ids[k]);
            need |= nd ? 1u << k : 0u;
            if (nd)
                load_sel<FMT>(src, ids[k], g0[k], g1[k]);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if ((need >> k) & 1u) {
                const float d = geom_score(g0[k], g1[k], X, Y, s);
                best.consider(ids[k], d, !(g0[k].x < 0.0f));
            }
        }
    }
    inject<FMT>(src, sc, seed_h, (uint32_t)row * (uint32_t)W + (uint32_t)col, n_slots, n_inject, X, Y, s, best);
    const long p = (long)row * W + col;
    store_list(cout, p, best.k);
}

// Propagation pass for jumps >= 5 on a per-pixel map (the pass of k_propagate:
// reading note, key design 3; summary, B.3), with the tile table sized for five
// regions.  Every lane holds its own list and its four lists at +-jump
// (for jump >= 16 these are four 16x16 blocks beside the tile; below that they
// overlap it) and their IDs go into an LDS hash table, so a distinct site's
// scoring record is gathered once per tile instead of once per candidate.  The
// hash has KT key slots for at most WTB = 512 records.  At jumps >= 16 (KT =
// WKT_SPARSE = 2048) the five regions name ~230 sites, and a wave repeats a CAS
// probe until its slowest lane has a slot, so a sparse table saves probes (by a
// simulation of converged lists, 1.7 CAS instructions per wave and list place
// at 2048 slots against 3.0 at 512); after the inserts a prefix scan gives each
// occupied key slot a record index, kept beside the records and read when an
// entry is scored; the keys and the compact ID list share their LDS with the
// records, which are written once they are dead.  At smaller jumps the regions
// overlap and name fewer sites: KT = WTB, the records sit at their key slots (no
// scan).  A tile whose own lists already name more
// than WIDE_OWN_MAX sites (random lists early in a cold start) would only
// overflow the table: it scores its neighbour candidates from their records, as
// the table-free pass does, and so do IDs beyond the table or the records.
constexpr int WKT_SPARSE = 2048;
constexpr int WTB = 512;
constexpr int WIDE_OWN_MAX = 96;
constexpr uint16_t WIDX_NONE = 0xFFFF;

template <int KT>
struct WideShared {
    union {
        struct {
            uint32_t key[KT];     // hash keys (site IDs)
            uint32_t recid[WTB];  // site ID of each record
        } h;
        struct {
            float4 rec0[WTB];     // scoring record, bytes 0..15
            float4 rec1[WTB];     // bytes 16..31; the site's ID in the last word
        } r;
    } u;
    uint16_t idx[KT > WTB ? KT : 1];  // record index of an occupied key slot (WIDX_NONE: beyond WTB)
    uint32_t wtot[BLOCK / 64];    // occupied key slots per wave's share (the scan)
    uint32_t n_own;               // distinct IDs of the tile's own lists

    // the record of table ref `ref` (< KT)
    __device__ __forceinline__ uint32_t rec_of(uint32_t ref) const
    {
        if constexpr (KT == WTB)
            return ref;
        else
            return idx[ref];
    }
};

// The records of a five-region (or 3x3) table once its inserts are done and a
// barrier has passed.  KT == WTB: one scoring record per occupied key slot, at
// its slot.  KT > WTB: a prefix scan numbers the occupied key slots (idx, kept
// beside the records: refs stay key slots and are looked up when scored), and one
// record per site is gathered; only in a tile with more sites than records are
// the refs of IDs beyond the last record turned into spills (their ID read from
// the key).  Records are written over the keys after a barrier; ends with a
// barrier.  All threads of the block call it.
template <int FMT, int KT, int NL, int NE>
__device__ __forceinline__ void table_records(WideShared<KT> &L, const SiteSrc &src, uint32_t (&refs)[NL][NE])
{
    const int tid = threadIdx.x;
    if constexpr (KT == WTB) {
        // one scoring record per occupied slot, at its slot, two slots per lane
        uint32_t c[WTB / BLOCK];
        float4 g0[WTB / BLOCK], g1[WTB / BLOCK];
#pragma unroll
        for (int j = 0; j < WTB / BLOCK; ++j) {
            c[j] = L.u.h.key[tid + j * BLOCK];
            g0[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            g1[j] = g0[j];
            if (c[j] != NONE)
                load_sel<FMT>(src, c[j], g0[j], g1[j]);
            g1[j].w = __uint_as_float(c[j]);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < WTB / BLOCK; ++j) {
            if (c[j] != NONE) {
                L.u.r.rec0[tid + j * BLOCK] = g0[j];
                L.u.r.rec1[tid + j * BLOCK] = g1[j];
            }
        }
    } else {
        // record indices: thread t takes key slots 8t .. 8t + 7; the occupied ones are
        // numbered in slot order by a wave scan and the waves' totals
        constexpr int KPT = KT / BLOCK;
        uint32_t occ = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            occ |= (L.u.h.key[KPT * tid + j] != NONE ? 1u : 0u) << j;
        const uint32_t cnt = __builtin_popcount(occ);
        const uint32_t incl = wave_incl_scan(cnt);
        if ((tid & 63) == 63)
            L.wtot[tid >> 6] = incl;
        __syncthreads();
        uint32_t base = incl - cnt, n_rec = 0;
#pragma unroll
        for (int w = 0; w < BLOCK / 64; ++w) {
            base += w < (tid >> 6) ? L.wtot[w] : 0u;
            n_rec += L.wtot[w];
        }
        n_rec = min(n_rec, (uint32_t)WTB);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if ((occ >> j) & 1u) {
                const uint32_t sl = KPT * tid + j;
                L.idx[sl] = base < (uint32_t)WTB ? (uint16_t)base : WIDX_NONE;
                if (base < (uint32_t)WTB)
                    L.u.h.recid[base] = L.u.h.key[sl];
                ++base;
            }
        }
        __syncthreads();
        // one scoring record per site, two per lane, gathered (and written over
        // the keys after the barrier); refs of IDs beyond the records become spills
        {
            if (n_rec == (uint32_t)WTB) {  // the block agrees: wtot is shared
#pragma unroll
                for (int li = 0; li < NL; ++li) {
#pragma unroll
                    for (int k = 0; k < NE; ++k) {
                        const uint32_t ref = refs[li][k];
                        if (ref < (uint32_t)KT && L.idx[ref] == WIDX_NONE)
                            refs[li][k] = REF_SPILL | L.u.h.key[ref];
                    }
                }
            }
            uint32_t c[WTB / BLOCK];
            float4 g0[WTB / BLOCK], g1[WTB / BLOCK];
#pragma unroll
            for (int j = 0; j < WTB / BLOCK; ++j) {
                const uint32_t r = tid + j * BLOCK;
                c[j] = r < n_rec ? L.u.h.recid[r] : NONE;
                g0[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                g1[j] = g0[j];
                if (c[j] != NONE)
                    load_sel<FMT>(src, c[j], g0[j], g1[j]);
                g1[j].w = __uint_as_float(c[j]);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < WTB / BLOCK; ++j) {
                if (c[j] != NONE) {
                    L.u.r.rec0[tid + j * BLOCK] = g0[j];
                    L.u.r.rec1[tid + j * BLOCK] = g1[j];
                }
            }
        }
    }
    __syncthreads();
}

template <int FMT, int KT>
__global__ __launch_bounds__(BLOCK) void k_propagate_wide(SiteSrc src, Screen sc, uint32_t n_slots,
                                                          const uint4 *__restrict__ cin, uint4 *__restrict__ cout,
                                                          int W, int H, int jump, uint32_t seed_h, int n_inject,
                                                          float s, int tiles_x, int nb)
{
    static_assert(KT == WTB || KT == WKT_SPARSE, "key table");
    __shared__ WideShared<KT> L;
    const int tid = threadIdx.x;
    const int t = xcd_band(blockIdx.x, nb);
    const int col = (t % tiles_x) * TILE + (tid & (TILE - 1));
    const int row = (t / tiles_x) * TILE + tid / TILE;
    const bool inside = col < W && row < H;
    for (int sl = tid; sl < KT; sl += BLOCK)
        L.u.h.key[sl] = NONE;
    if (tid == 0)
        L.n_own = 0u;
    // The five lists: own, then left, right, top and bottom (NONE outside the
    // image).  Neighbouring pixels hold the same sites at the same list places,
    // and CAS instructions whose lanes name one LDS address serialise (about two
    // cycles per lane on gfx950, against ~15 cycles for a wave on spread
    // addresses), so odd lanes take the two 16-byte halves of each list in the
    // other order: the lanes of one CAS then name one address less often.
    // Scoring and selection do not depend on the order.
    uint32_t ids[5][K];
    const int h = tid & 1;
#pragma unroll
    for (int li = 0; li < 5; ++li) {
        const int c = li == 1 ? col - jump : li == 2 ? col + jump : col;
        const int r = li == 3 ? row - jump : li == 4 ? row + jump : row;
        uint4 a = make_uint4(NONE, NONE, NONE, NONE), b = a;
        if (inside && c >= 0 && c < W && r >= 0 && r < H) {
            const long q = (long)r * W + c;
            a = cin[2 * q + h];
            b = cin[2 * q + 1 - h];
        }
        ids[li][0] = a.x; ids[li][1] = a.y; ids[li][2] = a.z; ids[li][3] = a.w;
        ids[li][4] = b.x; ids[li][5] = b.y; ids[li][6] = b.z; ids[li][7] = b.w;
    }
    __syncthreads();
    uint32_t refs[5][K];
    table_insert_ids<KT, K, true>(L.u.h.key, ids[0], n_slots, refs[0], &L.n_own);
    __syncthreads();
    const bool coherent = L.n_own <= (uint32_t)WIDE_OWN_MAX;
    if (coherent) {
#pragma unroll
        for (int li = 1; li < 5; ++li)
            table_insert_ids<KT, K>(L.u.h.key, ids[li], n_slots, refs[li]);
    } else {
#pragma unroll
        for (int li = 1; li < 5; ++li)
#pragma unroll
            for (int k = 0; k < K; ++k)
                refs[li][k] = ids[li][k] < n_slots ? (REF_SPILL | ids[li][k]) : REF_NONE;
    }
    __syncthreads();
    table_records<FMT, KT>(L, src, refs);
    if (!inside)
        return;
    const float X = (float)col + 0.5f, Y = (float)row + 0.5f;
    TopK64 best;
    // own list: its table entries (an ID the list repeats keeps its first place
    // only), sorted with the network; then entries the table could not hold
    {
        uint64_t v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t ref = refs[0][k];
            bool dup = false;
#pragma unroll
            for (int j = 0; j < k; ++j)
                dup |= refs[0][j] == ref;
            v[k] = ~0ull;
            if (ref < (uint32_t)KT && !dup) {
                const uint32_t rr = L.rec_of(ref);
                const float4 g0 = L.u.r.rec0[rr], g1 = L.u.r.rec1[rr];
                const float d = geom_score(g0, g1, X, Y, s);
                if (!(g0.x < 0.0f) && finitef(d))
                    v[k] = rank_key(d, __float_as_uint(g1.w));
            }
        }
        best.set_sorted(v);
    }
    // the neighbour lists (their IDs may repeat the list's: consider() checks),
    // and every entry the table does not hold, from its record in global memory
#pragma unroll
    for (int li = 0; li < 5; ++li) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t ref = refs[li][k];
            if (ref < (uint32_t)KT) {
                if (li > 0) {
                    const uint32_t rr = L.rec_of(ref);
                    const float4 g0 = L.u.r.rec0[rr], g1 = L.u.r.rec1[rr];
                    best.consider(__float_as_uint(g1.w), geom_score(g0, g1, X, Y, s), !(g0.x < 0.0f));
                }
            } else if (ref != REF_NONE) {
                const uint32_t c = ref & ~REF_SPILL;
                if (!best.holds(c)) {
                    bool usable;
                    const float d = geom_score_id<FMT>(src, c, X, Y, s, usable);
                    best.consider_new(c, d, usable);
                }
            }
        }
    }
    inject<FMT>(src, sc, seed_h, (uint32_t)row * (uint32_t)W + (uint32_t)col, n_slots, n_inject, X, Y, s, best);
    store_list(cout, (long)row * W + col, best.k);
}

// ---------------------------------------------------------------------------
// Jump-flood prepass (summary, Appendix B.3 "Jump schedule": an optional prepass
// for (re)initialisation -- a seed pass, then ceil(log2 max(W, H)) flood passes
// over 3x3 neighbourhoods that keep the four closest sites).
//
// Seed: every active site with a finite position enters the list of the map
// entry of the pixel that contains it; an entry keeps at most four, the best by
// (d, ID) at its centred UV.  On the GPU the four places are filled in four rounds (one launch
// each): in round r every site not already in places 0..r-1 offers its 64-bit
// ranking key to place r with an atomic minimum, so place r ends up with the
// r-th best key whatever the order of arrival.  The places are the four 8-byte
// pairs of the pixel's 32-byte list; a last pass turns keys into IDs.
constexpr int JFA_KEEP = 4;

__global__ __launch_bounds__(256) void k_fill_map(uint4 *__restrict__ cand, long n4)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n4)
        cand[i] = make_uint4(NONE, NONE, NONE, NONE);
}

// Seeding pairs (entry, ID), grouped by entry and in write order within an
// entry: the first pair of each group applies the group's pairs in order, each
// writing its ID into the last place of the entry's list unless the list holds
// it already (the lists keep distinct IDs).
__global__ __launch_bounds__(256) void k_apply_seeds(uint32_t *__restrict__ cand, long n_entries,
                                                     const uint2 *__restrict__ seeds, long n_seeds)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_seeds)
        return;
    const uint32_t e = seeds[i].x;
    if (i > 0 && seeds[i - 1].x == e)
        return;  // not the first pair of its group
    if ((long)e >= n_entries)
        return;
    uint32_t *L = cand + (size_t)e * K;
    for (long j = i; j < n_seeds && seeds[j].x == e; ++j) {
        const uint32_t id = seeds[j].y;
        bool held = false;
#pragma unroll
        for (int k = 0; k < K; ++k)
            held |= L[k] == id;
        if (!held)
            L[K - 1] = id;
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void k_jfa_seed_round(SiteSrc src, uint32_t n_slots,
                                                        unsigned long long *__restrict__ keys, int W, int H,
                                                        float s, MapGrid mg, int round)
{
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n_slots)
        return;
    float4 g0, g1;
    load_sel<FMT>(src, i, g0, g1);
    if (!(g0.x >= 0.0f) || !finitef(g0.x) || !finitef(g0.y))
        return;  // inactive (x < 0), or no position
    // the map entry of the pixel that holds the site
    const int col = (int)floorf(fminf(g0.x, (float)(W - 1))) / mg.c;
    const int row = (int)floorf(fminf(fmaxf(g0.y, 0.0f), (float)(H - 1))) / mg.c;
    const float d = geom_score(g0, g1, ((float)col + 0.5f) * mg.sx, ((float)row + 0.5f) * mg.sy, s);
    if (!finitef(d))
        return;
    const unsigned long long key = rank_key(d, i);
    unsigned long long *pl = keys + ((size_t)row * mg.Wm + col) * JFA_KEEP;
    for (int r = 0; r < round; ++r)
        if (pl[r] == key)
            return;  // already placed
    atomicMin(pl + round, key);
}

// keys -> IDs: the low word of a key is the site's ID (the sentinel where no key
// arrived); entries 4..7 are the sentinel.
__global__ __launch_bounds__(256) void k_jfa_seed_finish(uint4 *__restrict__ cand, long P)
{
    const long p = (long)blockIdx.x * 256 + threadIdx.x;
    if (p >= P)
        return;
    const uint4 a = cand[2 * p], b = cand[2 * p + 1];
    cand[2 * p] = make_uint4(a.x, a.z, b.x, b.z);
    cand[2 * p + 1] = make_uint4(NONE, NONE, NONE, NONE);
}

// One flood pass with step `step`: the union of the first four entries of the 3x3
// lists at offsets {-step, 0, step}^2 inside the image; the four best by (d, ID)
// go to entries 0..3, the sentinel to 4..7.  Table-free: candidates are scored
// straight from their records (an ID already held is skipped first).  Screening
// candidates against the fourth place, the entry's own list first, was measured
// slower: at steps 16-256 the fourth place is still far, few candidates are
// dropped and every one costs a screen-word gather on top of its record
// (4096x4096 after an edit: 3.8-5.0 vs 2.9-3.9 ms per pass).
template <int FMT>
__global__ __launch_bounds__(BLOCK) void k_jfa_pass(SiteSrc src, uint32_t n_slots,
                                                    const uint4 *__restrict__ cin, uint4 *__restrict__ cout, int W,
                                                    int H, int step, float s, float sx, float sy, int tiles_x,
                                                    int nb)
{
    const int t = xcd_band(blockIdx.x, nb);
    const int col = (t % tiles_x) * TILE + (threadIdx.x & (TILE - 1));
    const int row = (t / tiles_x) * TILE + (threadIdx.x / TILE);
    if (col >= W || row >= H)
        return;
    const float X = ((float)col + 0.5f) * sx, Y = ((float)row + 0.5f) * sy;
    TopK64 best;
#pragma unroll
    for (int j = 0; j < K; ++j)
        best.k[j] = ~0ull;
    for (int li = 0; li < 9; ++li) {
        const int c = col + (li % 3 - 1) * step, r = row + (li / 3 - 1) * step;
        if (c < 0 || c >= W || r < 0 || r >= H)
            continue;
        const uint4 a = cin[2 * ((long)r * W + c)];
        const uint32_t ids[JFA_KEEP] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < JFA_KEEP; ++k) {
            if (ids[k] < n_slots && !best.holds(ids[k])) {
                bool usable;
                const float d = geom_score_id<FMT>(src, ids[k], X, Y, s, usable);
                best.consider_new(ids[k], d, usable);
            }
        }
    }
    const long p = (long)row * W + col;
    cout[2 * p] = make_uint4((uint32_t)best.k[0], (uint32_t)best.k[1], (uint32_t)best.k[2], (uint32_t)best.k[3]);
    cout[2 * p + 1] = make_uint4(NONE, NONE, NONE, NONE);
}

// The same flood pass on a per-pixel map through a tile table: at small steps the
// nine lists of neighbouring pixels name mostly the same sites, so their IDs go into the
// sparse hash of the five-region table (2048 key slots, 512 records) and each
// distinct site's scoring record is gathered once per tile; candidates are
// scored from the LDS records, IDs beyond the table from their global records.
// The candidates and the selection are those of k_jfa_pass.
template <int FMT>
__global__ __launch_bounds__(BLOCK) void k_jfa_pass_table(SiteSrc src, uint32_t n_slots,
                                                          const uint4 *__restrict__ cin, uint4 *__restrict__ cout,
                                                          int W, int H, int step, float s, int tiles_x, int nb)
{
    __shared__ WideShared<WKT_SPARSE> L;
    const int tid = threadIdx.x;
    const int t = xcd_band(blockIdx.x, nb);
    const int col = (t % tiles_x) * TILE + (tid & (TILE - 1));
    const int row = (t / tiles_x) * TILE + tid / TILE;
    const bool inside = col < W && row < H;
    for (int sl = tid; sl < WKT_SPARSE; sl += BLOCK)
        L.u.h.key[sl] = NONE;
    __syncthreads();
    uint32_t refs[9][JFA_KEEP];
#pragma unroll
    for (int li = 0; li < 9; ++li) {
        const int c = col + (li % 3 - 1) * step, r = row + (li / 3 - 1) * step;
        uint4 a = make_uint4(NONE, NONE, NONE, NONE);
        if (inside && c >= 0 && c < W && r >= 0 && r < H)
            a = cin[2 * ((long)r * W + c)];
        const uint32_t ids[JFA_KEEP] = {a.x, a.y, a.z, a.w};
        table_insert_ids<WKT_SPARSE, JFA_KEEP>(L.u.h.key, ids, n_slots, refs[li]);
    }
    __syncthreads();
    table_records<FMT, WKT_SPARSE>(L, src, refs);
    if (!inside)
        return;
    const float X = (float)col + 0.5f, Y = (float)row + 0.5f;
    TopK64 best;
#pragma unroll
    for (int j = 0; j < K; ++j)
        best.k[j] = ~0ull;
#pragma unroll
    for (int li = 0; li < 9; ++li) {
#pragma unroll
        for (int k = 0; k < JFA_KEEP; ++k) {
            const uint32_t ref = refs[li][k];
            if (ref < (uint32_t)WKT_SPARSE) {
                const uint32_t rr = L.rec_of(ref);
                const float4 g0 = L.u.r.rec0[rr], g1 = L.u.r.rec1[rr];
                best.consider(__float_as_uint(g1.w), geom_score(g0, g1, X, Y, s), !(g0.x < 0.0f));
            } else if (ref != REF_NONE) {
                const uint32_t c = ref & ~REF_SPILL;
                if (!best.holds(c)) {
                    bool usable;
                    const float d = geom_score_id<FMT>(src, c, X, Y, s, usable);
                    best.consider_new(c, d, usable);
                }
            }
        }
    }
    const long p = (long)row * W + col;
    cout[2 * p] = make_uint4((uint32_t)best.k[0], (uint32_t)best.k[1], (uint32_t)best.k[2], (uint32_t)best.k[3]);
    cout[2 * p + 1] = make_uint4(NONE, NONE, NONE, NONE);
}

// ---------------------------------------------------------------------------
// Exact top-K by brute force: every slot is scored for every pixel.  Scoring
// records are staged through LDS 256 at a time.
template <int FMT>
__global__ __launch_bounds__(BLOCK) void k_topk_exact(SiteSrc src, uint32_t n_slots,
                                                      uint4 *__restrict__ cout, int W, int H, float s, float sx,
                                                      float sy, int tiles_x, int nb)
{
    __shared__ float4 l0[BLOCK], l1[BLOCK];
    const int t = xcd_band(blockIdx.x, nb);
    const int col = (t % tiles_x) * TILE + (threadIdx.x & (TILE - 1));
    const int row = (t / tiles_x) * TILE + (threadIdx.x / TILE);
    const bool inside = col < W && row < H;
    const float X = ((float)col + 0.5f) * sx, Y = ((float)row + 0.5f) * sy;
    TopK64 best;
#pragma unroll
    for (int j = 0; j < K; ++j)
        best.k[j] = ~0ull;
    for (uint32_t base = 0; base < n_slots; base += BLOCK) {
        const uint32_t i = base + threadIdx.x;
        float4 g0 = make_float4(-1.0f, 0.0f, 0.0f, 0.0f), g1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (i < n_slots)
            load_sel<FMT>(src, i, g0, g1);
        __syncthreads();
        l0[threadIdx.x] = g0;
        l1[threadIdx.x] = g1;
        __syncthreads();
        if (inside) {
            const int cnt = min((int)(n_slots - base), BLOCK);
            for (int j = 0; j < cnt; ++j) {
                const float4 a0 = l0[j];
                const float d = geom_score(a0, l1[j], X, Y, s);
                best.consider_new(base + j, d, !(a0.x < 0.0f));
            }
        }
    }
    if (inside) {
        const long p = (long)row * W + col;
        cout[2 * p] = make_uint4((uint32_t)best.k[0], (uint32_t)best.k[1], (uint32_t)best.k[2], (uint32_t)best.k[3]);
        cout[2 * p + 1] =
            make_uint4((uint32_t)best.k[4], (uint32_t)best.k[5], (uint32_t)best.k[6], (uint32_t)best.k[7]);
    }
}

// Exact top-K at chosen map entries (entry index row * Wm + col each), for recall
// measurements on maps too large for the whole-map brute force: one entry per
// lane, every slot scored, scoring records staged through LDS as above.
template <int FMT>
__global__ __launch_bounds__(BLOCK) void k_topk_exact_at(SiteSrc src, uint32_t n_slots,
                                                         const uint32_t *__restrict__ ent, int n_ent,
                                                         uint4 *__restrict__ out, int Wm, int Hm, float s,
                                                         float sx, float sy)
{
    __shared__ float4 l0[BLOCK], l1[BLOCK];
    const int q = blockIdx.x * BLOCK + threadIdx.x;
    const bool inside = q < n_ent;
    uint32_t e = inside ? ent[q] : 0u;
    const bool valid = inside && e < (uint32_t)Wm * (uint32_t)Hm;
    e = valid ? e : 0u;
    const int col = (int)(e % (uint32_t)Wm), row = (int)(e / (uint32_t)Wm);
    const float X = ((float)col + 0.5f) * sx, Y = ((float)row + 0.5f) * sy;
    TopK64 best;
#pragma unroll
    for (int j = 0; j < K; ++j)
        best.k[j] = ~0ull;
    for (uint32_t base = 0; base < n_slots; base += BLOCK) {
        const uint32_t i = base + threadIdx.x;
        float4 g0 = make_float4(-1.0f, 0.0f, 0.0f, 0.0f), g1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (i < n_slots)
            load_sel<FMT>(src, i, g0, g1);
        __syncthreads();
        l0[threadIdx.x] = g0;
        l1[threadIdx.x] = g1;
        __syncthreads();
        if (valid) {
            const int cnt = min((int)(n_slots - base), BLOCK);
            for (int j = 0; j < cnt; ++j) {
                const float4 a0 = l0[j];
                const float d = geom_score(a0, l1[j], X, Y, s);
                best.consider_new(base + j, d, !(a0.x < 0.0f));
            }
        }
    }
    if (inside) {
        out[2 * (long)q] = make_uint4((uint32_t)best.k[0], (uint32_t)best.k[1], (uint32_t)best.k[2],
                                      (uint32_t)best.k[3]);
        out[2 * (long)q + 1] = make_uint4((uint32_t)best.k[4], (uint32_t)best.k[5], (uint32_t)best.k[6],
                                          (uint32_t)best.k[7]);
    }
}

// ---------------------------------------------------------------------------
// Per-tile site table.  A 16x16 tile's lists name only a few dozen distinct
// sites, so each distinct site is gathered once per tile and its derived record
// kept in LDS: scattered per-lane gathers are what limits these kernels
// otherwise.  The table is an LDS hash keyed by site ID (the summary's B.4 per-
// tile hash: multiplicative hash with double hashing, <= HASH_PROBES probes, one
// CAS per probe; table_insert_ids).  An ID that finds no slot takes the "spill"
// path and is read from global memory.
constexpr int TBL = 256;
constexpr int NREC = 12;  // (px py r tau) (ux uy E iE) (R G B inv_n): three float4

enum { R_PX, R_PY, R_R, R_TAU, R_UX, R_UY, R_E, R_IE, R_C0, R_C1, R_C2, R_INVN };

// Derived record of one site: the metric frame, tau = exp(log tau), the colour
// and 1/|dir| (0 for a degenerate direction).  A site that cannot take part --
// inactive (x < 0, summary B.2) or with a non-finite colour -- gets px = NaN, so
// every logit it produces is non-finite and the entry is dropped.
struct SiteRec {
    float v[NREC];
};

// Render record of site c from its 64-byte record (FMT = SEL_REC) or from the
// planes (SEL_SOA: the same derivation as make_record_v, so the same bits).
template <int FMT>
__device__ __forceinline__ SiteRec load_rec_global(const SiteSrc &src, uint32_t c)
{
    float4 a, b, cc, d;
    if constexpr (FMT == SEL_SOA) {
        float p[SAD_NPARAM];
#pragma unroll
        for (int k = 0; k < SAD_NPARAM; ++k)
            p[k] = src.S[k * src.st + c];
        float4 o[RLD4];
        make_record_v(p, o);
        a = o[0];
        b = o[1];
        cc = o[2];
        d = o[3];
    } else {
        static_assert(FMT == SEL_REC, "render kernels read records or planes");
        const float4 *G = src.G;
        a = G[RLD4 * (size_t)c];
        b = G[RLD4 * (size_t)c + 1];
        cc = G[RLD4 * (size_t)c + 2];
        d = G[RLD4 * (size_t)c + 3];
    }
    SiteRec R;
    // an inactive site or one with a non-finite colour is unusable: px = NaN makes
    // its score NaN, and its colour is 0 so that a zero weight times it adds 0
    const bool ok = !(a.x < 0.0f) && finitef(cc.x) && finitef(cc.y) && finitef(cc.z);
    R.v[R_PX] = ok ? a.x : __builtin_nanf("");
    R.v[R_PY] = a.y;
    R.v[R_R] = a.z;
    R.v[R_UX] = d.x;
    R.v[R_UY] = d.y;
    R.v[R_E] = d.z;
    R.v[R_IE] = d.w;
    R.v[R_TAU] = b.w;
    R.v[R_C0] = ok ? cc.x : 0.0f;
    R.v[R_C1] = ok ? cc.y : 0.0f;
    R.v[R_C2] = ok ? cc.z : 0.0f;
    R.v[R_INVN] = cc.w;
    return R;
}

// Records are kept slot-major as three float4, so a lane fetches a record with
// three 16-byte LDS reads rather than one read per field.
struct TileTable {
    uint32_t key[TBL];
    float4 rec[TBL + 1][NREC / 4];  // slot TBL: the null record (px = NaN) for empty entries
};

// Phases 1-2 shared by forward and backward: insert the pixel's IDs, then one
// thread per occupied slot fills its record.  slot[k]: table slot, -1 = spill,
// -2 = no site (sentinel or ID >= n_slots).  Ends with a barrier.
__device__ __forceinline__ void table_insert_phase(TileTable &T, uint32_t n_slots, const uint32_t (&ids)[K],
                                                   int (&slot)[K])
{
    T.key[threadIdx.x] = NONE;
    __syncthreads();
    uint32_t refs[K];
    table_insert_ids<TBL>(T.key, ids, n_slots, refs);
#pragma unroll
    for (int k = 0; k < K; ++k)
        slot[k] = refs[k] == REF_NONE ? -2 : (refs[k] & REF_SPILL) ? -1 : (int)refs[k];
}

// One thread per slot: the slot's record (after a barrier that completes the
// inserts), and the null record.  Ends with a barrier.
template <int FMT>
__device__ __forceinline__ void table_load_phase(TileTable &T, const SiteSrc &src)
{
    const uint32_t c = T.key[threadIdx.x];
    if (c != NONE) {
        const SiteRec R = load_rec_global<FMT>(src, c);
#pragma unroll
        for (int j = 0; j < NREC / 4; ++j)
            T.rec[threadIdx.x][j] = make_float4(R.v[4 * j], R.v[4 * j + 1], R.v[4 * j + 2], R.v[4 * j + 3]);
    }
    if (threadIdx.x < NREC / 4)
        T.rec[TBL][threadIdx.x] = make_float4(threadIdx.x == 0 ? __builtin_nanf("") : 0.0f, 0.0f, 0.0f, 0.0f);
    __syncthreads();
}

template <int FMT>
__device__ __forceinline__ void build_tile_table(TileTable &T, const SiteSrc &src, uint32_t n_slots,
                                                 const uint32_t (&ids)[K], int (&slot)[K])
{
    table_insert_phase(T, n_slots, ids, slot);
    __syncthreads();
    table_load_phase<FMT>(T, src);
}

__device__ __forceinline__ SiteRec table_rec(const TileTable &T, int sl)
{
    SiteRec R;
#pragma unroll
    for (int j = 0; j < NREC / 4; ++j) {
        const float4 q = T.rec[sl][j];
        R.v[4 * j] = q.x;
        R.v[4 * j + 1] = q.y;
        R.v[4 * j + 2] = q.z;
        R.v[4 * j + 3] = q.w;
    }
    return R;
}

__device__ __forceinline__ float rec_score(const SiteRec &R, float X, float Y, float s)
{
    const Frame f{R.v[R_UX], R.v[R_UY], R.v[R_E], R.v[R_IE]};
    return score_frame(f, R.v[R_PX], R.v[R_PY], R.v[R_R], X, Y, s);
}

// The blend of one pixel's list (reading note, key design 2; summary B.4:
// max-subtracted softmax, invalid and non-finite entries skipped).
struct PixelBlend {
    float l[K], e[K], c0[K], c1[K], c2[K];
    bool use[K];
    float Z, chat0, chat1, chat2;
    bool any;
};


// Record of list entry k: from the tile table, from global memory for a spilled
// ID, or an unusable placeholder (px = NaN) for an empty entry.
template <int FMT>
__device__ __forceinline__ SiteRec fetch_rec(const TileTable &T, const SiteSrc &src, uint32_t id, int sl)
{
    if (sl >= 0)
        return table_rec(T, sl);
    if (sl == -1)
        return load_rec_global<FMT>(src, id);
    SiteRec R;
#pragma unroll
    for (int j = 0; j < NREC; ++j)
        R.v[j] = 0.0f;
    R.v[R_PX] = __builtin_nanf("");
    return R;
}

template <int FMT>
__device__ __forceinline__ void blend_pixel(const TileTable &T, const SiteSrc &src,
                                            const uint32_t (&ids)[K], const int (&slot)[K], float X, float Y,
                                            float s, PixelBlend &B)
{
    // every entry reads the table (empty and spilled ones the null record), then
    // spilled entries, if the wave has any, are redone from their global records
    auto entry = [&](int k, const SiteRec &R) {
        const float l = -R.v[R_TAU] * rec_score(R, X, Y, s);
        B.use[k] = finitef(l);
        B.l[k] = l;
        // finite (0 for an unusable record); an entry not used gets weight 0
        B.c0[k] = R.v[R_C0];
        B.c1[k] = R.v[R_C1];
        B.c2[k] = R.v[R_C2];
    };
    bool spilled = false;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        entry(k, table_rec(T, slot[k] >= 0 ? slot[k] : TBL));
        spilled |= slot[k] == -1;
    }
    if (__any(spilled)) {
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (slot[k] == -1)
                entry(k, load_rec_global<FMT>(src, ids[k]));
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < K; ++k)
        mx = B.use[k] ? fmaxf(mx, B.l[k]) : mx;
    B.any = mx > -__builtin_inff();
    // entries 0..3 and 4..7 are summed separately and then added: the order of
    // the backward, whose two lanes per pixel each sum one half
    float Z = 0.0f, a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, Zb = 0.0f, b0 = 0.0f, b1 = 0.0f, b2 = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float e = B.use[k] ? __expf(B.l[k] - mx) : 0.0f;
        B.e[k] = e;
        if (k < K / 2) {
            Z += e;
            a0 = fmaf(e, B.c0[k], a0);
            a1 = fmaf(e, B.c1[k], a1);
            a2 = fmaf(e, B.c2[k], a2);
        } else {
            Zb += e;
            b0 = fmaf(e, B.c0[k], b0);
            b1 = fmaf(e, B.c1[k], b1);
            b2 = fmaf(e, B.c2[k], b2);
        }
    }
    Z += Zb;
    a0 += b0;
    a1 += b1;
    a2 += b2;
    B.Z = Z;
    const float iZ = B.any ? hw_rcp(Z) : 0.0f;  // Z >= 1: the largest term is exp(0)
    B.chat0 = a0 * iZ;
    B.chat1 = a1 * iZ;
    B.chat2 = a2 * iZ;
}

__device__ __forceinline__ void tile_pixel(int nb, int tiles_x, int &col, int &row)
{
    const int t = xcd_band(blockIdx.x, nb);
    col = (t % tiles_x) * TILE + (threadIdx.x & (TILE - 1));
    row = (t / tiles_x) * TILE + (threadIdx.x / TILE);
}

// The list of map entry p in the order in which place e holds entry e ^ m, m =
// 4h + 2r + t (the column's low three bits): neighbouring lanes then insert
// different list places into the tile table.  It is the order of the fused
// backward's lane pairs, so the forward's image matches the backward's bits.
__device__ __forceinline__ void load_ids(const uint4 *__restrict__ cand, long p, bool inside, uint32_t (&ids)[K],
                                         int h, int r, bool t)
{
    uint2 q4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        q4[j] = make_uint2(NONE, NONE);
    if (inside) {
        const uint2 *q = reinterpret_cast<const uint2 *>(cand) + 4 * p;
        q4[0] = q[2 * h + r];
        q4[1] = q[2 * h + 1 - r];
        q4[2] = q[2 * (1 - h) + r];
        q4[3] = q[2 * (1 - h) + 1 - r];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ids[2 * j] = t ? q4[j].y : q4[j].x;
        ids[2 * j + 1] = t ? q4[j].x : q4[j].y;
    }
}


// Render forward (reading note, key design 2; project page "Method").
template <int FMT>
__global__ __launch_bounds__(BLOCK) void k_render_fwd(SiteSrc src, uint32_t n_slots,
                                                      const uint4 *__restrict__ cand, int W, int H,
                                                      float *__restrict__ out, float s, MapGrid mg, int tiles_x, int nb)
{
    __shared__ TileTable T;
    int col, row;
    tile_pixel(nb, tiles_x, col, row);
    const bool inside = col < W && row < H;
    const long p = (long)row * W + col;
    uint32_t ids[K];
    int slot[K];
    load_ids(cand, mg.entry(p, col, row), inside, ids, col & 1, (col >> 1) & 1, (col >> 2) & 1);
    build_tile_table<FMT>(T, src, n_slots, ids, slot);
    if (!inside)
        return;
    PixelBlend B;
    blend_pixel<FMT>(T, src, ids, slot, (float)col + 0.5f, (float)row + 0.5f, s, B);
    out[3 * p] = B.chat0;
    out[3 * p + 1] = B.chat1;
    out[3 * p + 2] = B.chat2;
}

// ---------------------------------------------------------------------------
// Render backward (summary, section 5 and B.4; press article section 5: 16x16
// tiles).  Per-entry gradients of L = sum ||c - t||^2, 11 accumulators per site
// (10 parameters + removal delta).
//
// The per-tile reduction avoids LDS float atomics (same-site entries of a tile
// collide on one address and serialise -- even one atomic per run of a site
// within a chunk of entries made the kernel more than twice as slow): entries
// are counting-sorted by table slot (one integer atomic per entry), each of 256
// threads then sums a fixed chunk of 8 sorted entries -- runs of one site -- in
// registers, and one thread per site adds the chunk partials of its run and
// issues one global atomic per accumulator.  Runs that lie strictly inside a
// chunk are flushed by the chunk thread.  Either way a site gets one global
// atomic per accumulator per tile.
constexpr int CHUNK = 8;
static_assert((SAD_LOSS_SLOTS & (SAD_LOSS_SLOTS - 1)) == 0, "loss slots: a power of two");
constexpr int NSUM = 10;  // per-entry sums of the reduction (entry_sums)

// Staged entries are 16-byte records; sorted entry e lives at record
// e ^ ((e >> 4) & 7).  Lanes that write one bucket write consecutive entries,
// which stay in distinct bank groups; when every thread reads the j-th entry of
// its chunk (entry 8t + j, one 128-bit read per entry) the XOR with (t / 2) mod 8
// puts 16 consecutive lanes on 16 distinct 4-bank groups of the 64 banks.
__device__ __forceinline__ int stage_pos(uint32_t e) { return (int)(e ^ ((e >> 4) & 7u)); }

struct BwdShared {
    TileTable T;
    uint32_t cnt[TBL];
    uint32_t off[TBL];
    float4 g[BLOCK];  // per pixel: 2 (c - t), and 0
    union {
        struct {
            float4 ent[BLOCK * K];  // (pixel | slot << 8, w, gamma, rdelta) per staged entry
        } e;
        struct {
            float part[2 * NSUM][BLOCK];  // per chunk: [0,10) head partial, [10,20) tail partial
            float fin[SAD_NACC][TBL];     // per table slot: the tile's sums, then its 11 totals
        } r;
    } u;
    float wsum[2 * BLOCK / 64];
    uint8_t occ[TBL];  // the occupied slots, ascending (n_occ of them)
    uint32_t total;
    uint32_t nspill;
    uint32_t n_occ;
};

// The backward of one site over a set of entries is linear in ten per-entry
// sums (derivation: reading note, key designs 1-2; alpha = u.delta,
// beta = u x delta, q^2 = e^a alpha^2 + e^-a beta^2, t = gamma / q, 0 at q = 0):
//   [0..2] w g   [3] gamma   [4] t alpha   [5] t beta   [6] t alpha^2
//   [7] t beta^2   [8] t alpha beta   [9] removal delta
// so the reduction adds these and site_grads turns a site's totals into its 11
// gradient contributions once.  Non-finite sums of an entry are dropped.
__device__ __forceinline__ void entry_sums(const SiteRec &R, float X, float Y, float w, float gamma, float rdelta,
                                           const float4 &g, float (&v)[NSUM])
{
    const float ex = X - R.v[R_PX], ey = Y - R.v[R_PY];
    const float ux = R.v[R_UX], uy = R.v[R_UY];
    const float al = ux * ex + uy * ey, be = ux * ey - uy * ex;
    const float q2 = R.v[R_E] * al * al + R.v[R_IE] * be * be;
    const float t = q2 > 0.0f ? gamma * __builtin_amdgcn_rsqf(q2) : 0.0f;
    const float tal = t * al, tbe = t * be;
    v[0] = w * g.x;
    v[1] = w * g.y;
    v[2] = w * g.z;
    v[3] = gamma;
    v[4] = tal;
    v[5] = tbe;
    v[6] = tal * al;
    v[7] = tbe * be;
    v[8] = tal * be;
    v[9] = rdelta;
    float all = v[0];
#pragma unroll
    for (int a = 1; a < NSUM; ++a)
        all += v[a];
    if (!finitef(all)) {
#pragma unroll
        for (int a = 0; a < NSUM; ++a)
            v[a] = finitef(v[a]) ? v[a] : 0.0f;
    }
}

// entry_sums added straight into a run's sums (multiply-adds), without the
// per-entry check for non-finite sums: the caller checks the run's totals and, if
// one is not finite, redoes the run with entry_sums.
__device__ __forceinline__ void entry_acc(const SiteRec &R, float X, float Y, float w, float gamma, float rdelta,
                                          const float4 &g, float (&run)[NSUM])
{
    const float ex = X - R.v[R_PX], ey = Y - R.v[R_PY];
    const float ux = R.v[R_UX], uy = R.v[R_UY];
    const float al = ux * ex + uy * ey, be = ux * ey - uy * ex;
    const float q2 = R.v[R_E] * al * al + R.v[R_IE] * be * be;
    const float t = q2 > 0.0f ? gamma * __builtin_amdgcn_rsqf(q2) : 0.0f;
    const float tal = t * al, tbe = t * be;
    run[0] = fmaf(w, g.x, run[0]);
    run[1] = fmaf(w, g.y, run[1]);
    run[2] = fmaf(w, g.z, run[2]);
    run[3] += gamma;
    run[4] += tal;
    run[5] += tbe;
    run[6] = fmaf(tal, al, run[6]);
    run[7] = fmaf(tbe, be, run[7]);
    run[8] = fmaf(tal, be, run[8]);
    run[9] += rdelta;
}

// A site's 11 gradient contributions from its entry-sum totals v (entry_sums):
//   colour: v[0..2]        r: tau s v[3]      log tau: -tau s (e^a v[6] + e^-a v[7] - r v[3])
//   p: tau s (e^a u v[4] + e^-a (-u_y, u_x) v[5])      a: -tau s (e^a v[6] - e^-a v[7]) / 2
//   dir: the gradient w.r.t. u projected off u and divided by |dir|, which for a
//        unit u is tau s (e^a - e^-a) v[8] (u_y, -u_x) / |dir|
//   removal delta: v[9]
__device__ __forceinline__ void site_grads(const SiteRec &R, float s, const float (&v)[NSUM], float (&acc)[SAD_NACC])
{
    const float ts = R.v[R_TAU] * s, E = R.v[R_E], iE = R.v[R_IE], ux = R.v[R_UX], uy = R.v[R_UY];
    acc[PCR] = v[0];
    acc[PCG] = v[1];
    acc[PCB] = v[2];
    acc[PR] = ts * v[3];
    acc[PLT] = -ts * (E * v[6] + iE * v[7] - R.v[R_R] * v[3]);
    acc[PX] = ts * (E * ux * v[4] - iE * uy * v[5]);
    acc[PY] = ts * (E * uy * v[4] + iE * ux * v[5]);
    acc[PA] = -0.5f * ts * (E * v[6] - iE * v[7]);
    const float in = R.v[R_INVN];
    const float cd = in > 0.0f ? ts * (E - iE) * v[8] * in : 0.0f;
    acc[PDX] = uy * cd;
    acc[PDY] = -ux * cd;
    acc[10] = v[9];
#pragma unroll
    for (int a = 0; a < SAD_NACC; ++a)
        acc[a] = finitef(acc[a]) ? acc[a] : 0.0f;
}

// Gradient accumulators: one 64-byte record per site (GL_REC: site i's 11 sums
// at g[16 i .. 16 i + 10]) or eleven planes (GL_PLANES: accumulator a of site i
// at g[a * st + i]).
constexpr int GL_REC = 0, GL_PLANES = 1;

struct GradOut {
    float *g;
    long st;
};

template <int GL>
__device__ __forceinline__ float *grad_at(const GradOut &o, uint32_t id, int a)
{
    if constexpr (GL == GL_REC)
        return o.g + (size_t)id * SAD_GRAD_LD + a;
    else
        return o.g + (size_t)a * o.st + id;
}

// Gradients of one spilled entry per lane (id = NONE: none), flushed by the
// whole wave together: the 11 sums of each lane are staged in LDS and
// consecutive lanes take consecutive accumulators of one site, so an atomic
// instruction touches a few 64-byte records instead of one per lane.
template <int FMT, int GL>
__device__ __forceinline__ void spill_flush(const SiteSrc &src, uint32_t id, float X, float Y, float s,
                                            float w, float gm, float dl, const float4 &g, float *vals,
                                            const GradOut &grad, int lane)
{
    uint32_t *vid = reinterpret_cast<uint32_t *>(vals + 64 * SAD_NACC);
    float acc[SAD_NACC];
#pragma unroll
    for (int a = 0; a < SAD_NACC; ++a)
        acc[a] = 0.0f;
    if (id != NONE) {
        const SiteRec R = load_rec_global<FMT>(src, id);
        float v[NSUM];
        entry_sums(R, X, Y, w, gm, dl, g, v);
        site_grads(R, s, v, acc);
    }
#pragma unroll
    for (int a = 0; a < SAD_NACC; ++a)
        vals[lane * SAD_NACC + a] = acc[a];  // odd stride: no bank conflicts
    vid[lane] = id;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = lane; i < 64 * SAD_NACC; i += 64) {
        const int e = i / SAD_NACC, a = i - e * SAD_NACC;
        const uint32_t c = vid[e];
        const float v = vals[i];
        if (c != NONE && v != 0.0f)
            unsafeAtomicAdd(grad_at<GL>(grad, c, a), v);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Two lanes per pixel: lanes l and l + 32 of a wave share a pixel and take
// entries 0..3 and 4..7 of its list.  The softmax and the removal delta need
// sums over all 8 entries; each lane sums its half and one v_permlane32_swap
// gives both lanes the pair's total (the same bits on both: the two halves are
// added in either order, and float addition commutes) and the partner's half.
// Per 16x16 tile this runs 8 waves over the same LDS as one lane per pixel, so a
// SIMD holds twice the waves to hide the latency of the table, record and
// staging phases, and each lane's serial chain of inserts and blends halves.
constexpr int PAIR_THREADS = 2 * BLOCK;
constexpr int KH = K / 2;

struct PairSums {
    float total, other;  // own half + partner's half; the partner's half
};

__device__ __forceinline__ PairSums pair_sums(float x, int half)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);  // lane l: x of lanes l % 32 and l % 32 + 32
    return {lo + hi, half ? lo : hi};
}

// The sum over each aligned group of 8 lanes, in every lane of the group: the
// partner across the pair (quad_perm [1,0,3,2]), across the quad ([2,3,0,1]),
// then across the half row (row_half_mirror: lane i of the 8 reads lane 7 - i,
// which lies in the other quad).  Three DPP moves, no LDS; the same additions in
// the same order as exchanging with lanes i^1, i^2, i^4.
__device__ __forceinline__ float group8_sum(float x)
{
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);  // row_half_mirror
    return x;
}

__device__ __forceinline__ float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The blend of one pixel's list over a lane pair (reading note, key design 2;
// summary B.4: max-subtracted softmax, invalid and non-finite entries skipped):
// this lane's half (entries 4 half .. 4 half + 3) and the pair's totals.  Every
// lane of the wave must take part (the exchanges read the partner lane).
struct PairBlend {
    float l[KH], e[KH], c0[KH], c1[KH], c2[KH];
    bool use[KH];
    bool any;
    PairSums Se, S0, S1, S2;  // sums of e and e c over the pair (and the partner's half)
    float iZ, chat0, chat1, chat2;
};

template <int FMT>
__device__ __forceinline__ void pair_blend(const TileTable &T, const SiteSrc &src,
                                           const uint32_t (&ids)[KH], const int (&slot)[KH], float X, float Y,
                                           float s, int half, PairBlend &B)
{
    // every entry reads the table (empty and spilled ones the null record), then
    // spilled entries, if the wave has any, are redone from their global records
    auto entry = [&](int k, const SiteRec &R) {
        const float lk = -R.v[R_TAU] * rec_score(R, X, Y, s);
        B.use[k] = finitef(lk);
        B.l[k] = lk;
        // finite (0 for an unusable record); an entry not used gets weight 0
        B.c0[k] = R.v[R_C0];
        B.c1[k] = R.v[R_C1];
        B.c2[k] = R.v[R_C2];
    };
    bool spilled = false;
#pragma unroll
    for (int k = 0; k < KH; ++k) {
        entry(k, table_rec(T, slot[k] >= 0 ? slot[k] : TBL));
        spilled |= slot[k] == -1;
    }
    if (__any(spilled)) {
#pragma unroll
        for (int k = 0; k < KH; ++k)
            if (slot[k] == -1)
                entry(k, load_rec_global<FMT>(src, ids[k]));
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < KH; ++k)
        mx = B.use[k] ? fmaxf(mx, B.l[k]) : mx;
    mx = pair_max(mx);
    B.any = mx > -__builtin_inff();
    float ze = 0.0f, z0 = 0.0f, z1 = 0.0f, z2 = 0.0f;
#pragma unroll
    for (int k = 0; k < KH; ++k) {
        B.e[k] = B.use[k] ? __expf(B.l[k] - mx) : 0.0f;
        ze += B.e[k];
        z0 = fmaf(B.e[k], B.c0[k], z0);
        z1 = fmaf(B.e[k], B.c1[k], z1);
        z2 = fmaf(B.e[k], B.c2[k], z2);
    }
    B.Se = pair_sums(ze, half);
    B.S0 = pair_sums(z0, half);
    B.S1 = pair_sums(z1, half);
    B.S2 = pair_sums(z2, half);
    B.iZ = B.any ? hw_rcp(B.Se.total) : 0.0f;  // Z >= 1: the largest term is exp(0)
    B.chat0 = B.S0.total * B.iZ;
    B.chat1 = B.S1.total * B.iZ;
    B.chat2 = B.S2.total * B.iZ;
}


template <int FMT, int GL>
__global__ __launch_bounds__(PAIR_THREADS) void k_render_bwd(SiteSrc src, uint32_t n_slots,
                                                            const uint4 *__restrict__ cand,
                                                            const float *__restrict__ target, int W, int H,
                                                            GradOut grad, float *__restrict__ loss_sum,
                                                            uint32_t loss_mask, float *__restrict__ out_rgb, float s,
                                                            MapGrid grid, int tiles_x, int nb)
{
    __shared__ BwdShared L;
    const int tid = threadIdx.x;
    const int lane = tid & 63, half = lane >> 5;
    const int pp = (tid >> 6) * 32 + (lane & 31);  // pixel within the tile
    const int t = xcd_band(blockIdx.x, nb);
    const int col0 = (t % tiles_x) * TILE, row0 = (t / tiles_x) * TILE;
    const int col = col0 + (pp & (TILE - 1)), row = row0 + pp / TILE;
    const bool inside = col < W && row < H;
    const long p = (long)row * W + col;
    // The lane pair holds the pixel's two list halves, in the order in which
    // place e holds list entry e ^ (pp & 7): odd pixels put the second half in
    // the lower lane, and the 8-byte quarters and the IDs within them swap on
    // bits 1 and 2.  Neighbouring lanes, which hold the same sites at the same
    // list places, then insert and count different places in one instruction
    // (same-address LDS atomics serialise: 249 -> 236 us at 2048x2048).  The
    // standalone forward loads its lists in the same order, so the fused image
    // stays bit-identical to it; the gradients do not depend on the order beyond
    // float rounding.
    uint32_t ids[KH];
    {
        uint2 a = make_uint2(NONE, NONE), b = a;
        if (inside) {
            const uint2 *q = reinterpret_cast<const uint2 *>(cand) + 4 * grid.entry(p, col, row) +
                             2 * (half ^ (pp & 1));
            const int r = (pp >> 1) & 1;
            a = q[r];
            b = q[1 - r];
        }
        const bool t = (pp >> 2) & 1;
        ids[0] = t ? a.y : a.x;
        ids[1] = t ? a.x : a.y;
        ids[2] = t ? b.y : b.x;
        ids[3] = t ? b.x : b.y;
    }
    // the target is read now, so its latency overlaps the table build
    float t0 = 0.0f, t1 = 0.0f, t2 = 0.0f;
    if (inside) {
        t0 = target[3 * p];
        t1 = target[3 * p + 1];
        t2 = target[3 * p + 2];
    }
    if (tid < TBL) {
        L.T.key[tid] = NONE;
        L.cnt[tid] = 0;
    }
    if (tid == 0)
        L.nspill = 0;
    __syncthreads();
    int slot[KH];
    {
        uint32_t refs[KH];
        table_insert_ids<TBL>(L.T.key, ids, n_slots, refs);
#pragma unroll
        for (int k = 0; k < KH; ++k)
            slot[k] = refs[k] == REF_NONE ? -2 : (refs[k] & REF_SPILL) ? -1 : (int)refs[k];
    }
    // every entry with a table slot gets its place in the slot-sorted staging now
    // (a counting sort whose counts are complete at the next barrier), so the
    // blend below can write its entries without another block-wide step
    uint32_t pos[KH];
    uint32_t nsp = 0;
#pragma unroll
    for (int k = 0; k < KH; ++k) {
        pos[k] = slot[k] >= 0 ? atomicAdd(&L.cnt[slot[k]], 1u) : 0u;
        nsp += slot[k] == -1;
    }
    if (__any(nsp > 0) && lane == 0)
        atomicAdd(&L.nspill, 1u);
    __syncthreads();
    // wave 0 turns the slot counts into bucket offsets (4 slots per lane, then a
    // wave scan) and lists the occupied slots, while the first 256 threads fill the
    // slot records
    if (tid < 64) {
        const uint4 c4 = reinterpret_cast<const uint4 *>(L.cnt)[lane];
        const uint32_t s0 = c4.x, s1 = s0 + c4.y, s2 = s1 + c4.z, s3 = s2 + c4.w;
        const uint32_t n0 = c4.x > 0, n1 = n0 + (c4.y > 0), n2 = n1 + (c4.z > 0), n3 = n2 + (c4.w > 0);
        const uint32_t incl = wave_incl_scan(s3), nincl = wave_incl_scan(n3);
        const uint32_t base = incl - s3, nbase = nincl - n3;
        reinterpret_cast<uint4 *>(L.off)[lane] = make_uint4(base, base + s0, base + s1, base + s2);
        if (c4.x > 0)
            L.occ[nbase] = (uint8_t)(4 * lane);
        if (c4.y > 0)
            L.occ[nbase + n0] = (uint8_t)(4 * lane + 1);
        if (c4.z > 0)
            L.occ[nbase + n1] = (uint8_t)(4 * lane + 2);
        if (c4.w > 0)
            L.occ[nbase + n2] = (uint8_t)(4 * lane + 3);
        if (lane == 63) {
            L.total = incl;
            L.n_occ = nincl;
        }
    }
    if (tid < TBL) {
        const uint32_t c = L.T.key[tid];
        if (c != NONE) {
            const SiteRec R = load_rec_global<FMT>(src, c);
#pragma unroll
            for (int j = 0; j < NREC / 4; ++j)
                L.T.rec[tid][j] = make_float4(R.v[4 * j], R.v[4 * j + 1], R.v[4 * j + 2], R.v[4 * j + 3]);
        }
    } else if (tid < TBL + NREC / 4) {
        const int j = tid - TBL;  // the null record (px = NaN) of empty entries
        L.T.rec[TBL][j] = make_float4(j == 0 ? __builtin_nanf("") : 0.0f, 0.0f, 0.0f, 0.0f);
    }
    const bool tile_spills = L.nspill > 0;  // the same for the whole block
    __syncthreads();

    // phase 3: blend over the pair (every lane takes part in the exchanges; a
    // pixel outside the image has no usable entry), per-entry softmax quantities;
    // staged entries written in slot order, spilled entries flushed to global memory
    const float X = (float)col + 0.5f, Y = (float)row + 0.5f;
    PairBlend B;
    pair_blend<FMT>(L.T, src, ids, slot, X, Y, s, half, B);
    const float *c0 = B.c0, *c1 = B.c1, *c2 = B.c2, *e = B.e;
    const bool *use = B.use;
    const bool any = B.any;
    const PairSums &Se = B.Se, &S0 = B.S0, &S1 = B.S1, &S2 = B.S2;
    const float iZ = B.iZ, chat0 = B.chat0, chat1 = B.chat1, chat2 = B.chat2;
    float err = 0.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
    if (inside) {
        if (out_rgb && half == 0) {  // the forward of the same map, for free
            out_rgb[3 * p] = chat0;
            out_rgb[3 * p + 1] = chat1;
            out_rgb[3 * p + 2] = chat2;
        }
        const float r0 = chat0 - t0, r1 = chat1 - t1, r2 = chat2 - t2;
        err = r0 * r0 + r1 * r1 + r2 * r2;
        g0 = 2.0f * r0;
        g1 = 2.0f * r1;
        g2 = 2.0f * r2;
    }
    float wk[KH], gk[KH], dk[KH];
    bool spill[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k) {
        wk[k] = gk[k] = dk[k] = 0.0f;
        spill[k] = false;
    }
    if (any) {
        // exclusive sums of e and e*c over the other 7 entries (removal delta):
        // the partner's half plus this half's entries before and after k
        float xe[KH], x0[KH], x1[KH], x2[KH];
        float se = Se.other, s0 = S0.other, s1 = S1.other, s2 = S2.other;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            xe[k] = se;
            x0[k] = s0;
            x1[k] = s1;
            x2[k] = s2;
            se += e[k];
            s0 += e[k] * c0[k];
            s1 += e[k] * c1[k];
            s2 += e[k] * c2[k];
        }
        se = s0 = s1 = s2 = 0.0f;
#pragma unroll
        for (int k = KH - 1; k >= 0; --k) {
            xe[k] += se;
            x0[k] += s0;
            x1[k] += s1;
            x2[k] += s2;
            se += e[k];
            s0 += e[k] * c0[k];
            s1 += e[k] * c1[k];
            s2 += e[k] * c2[k];
        }
        // 1 / (sum of the other entries' e): xe >= 2^-100 but for near-exclusive
        // entries, which take the exact quotient (rarely: a wave-uniform branch)
        float iZo[KH];
        bool tiny = false;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            iZo[k] = xe[k] > 0.0f ? hw_rcp(xe[k]) : 0.0f;
            tiny |= xe[k] > 0.0f && xe[k] < 0x1p-100f;
        }
        if (__any(tiny)) {
#pragma unroll
            for (int k = 0; k < KH; ++k)
                if (xe[k] > 0.0f && xe[k] < 0x1p-100f)
                    iZo[k] = 1.0f / xe[k];
        }
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const float w = e[k] * iZ;
            // a zero-weight entry changes nothing: all its gradients vanish and
            // removing it leaves the blend as it is (it stays staged, as zeros)
            if (!use[k] || w == 0.0f)
                continue;
            wk[k] = w;
            gk[k] = w * (g0 * (c0[k] - chat0) + g1 * (c1[k] - chat1) + g2 * (c2[k] - chat2));
            const float m0 = x0[k] * iZo[k] - t0, m1 = x1[k] * iZo[k] - t1, m2 = x2[k] * iZo[k] - t2;
            dk[k] = (m0 * m0 + m1 * m1 + m2 * m2) - err;
            spill[k] = slot[k] == -1;
        }
    }
    auto stage_entries = [&]() {
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            if (slot[k] >= 0) {
                const int q = stage_pos(L.off[slot[k]] + pos[k]);
                L.u.e.ent[q] = make_float4(__uint_as_float((uint32_t)pp | ((uint32_t)slot[k] << 8)), wk[k], gk[k],
                                           dk[k]);
            }
        }
    };
    if (!tile_spills) {
        stage_entries();
    } else {
        // Spilled entries (IDs the tile table could not hold), k by k where any
        // lane of the wave has one (see spill_flush).  Their LDS staging shares the
        // sort's storage, so the tile stages its entries only after all waves are
        // done with it.
        float *vals = &L.u.r.part[0][0] + (tid >> 6) * (64 * SAD_NACC + 64);
#pragma unroll
        for (int k = 0; k < KH; ++k)
            if (__any(spill[k]))
                spill_flush<FMT, GL>(src, spill[k] ? ids[k] : NONE, X, Y, s, wk[k], gk[k], dk[k], make_float4(g0, g1, g2, 0.0f),
                            vals, grad, lane);
        __syncthreads();
        stage_entries();
    }
    if (half == 0)
        L.g[pp] = make_float4(g0, g1, g2, 0.0f);
    // per-pixel loss (counted once per pair): wave sums -- each 8-lane group by
    // DPP moves, then the eight group sums read from their first lanes
    {
        const float v = group8_sum(half == 0 ? err : 0.0f);
        float w = 0.0f;
#pragma unroll
        for (int g = 0; g < 8; ++g)
            w += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 8 * g));
        if (lane == 0)
            L.wsum[tid >> 6] = w;
    }
    __syncthreads();
    if (tid == 0 && loss_sum) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < PAIR_THREADS / 64; ++w)
            v += L.wsum[w];
        unsafeAtomicAdd(loss_sum + (blockIdx.x & loss_mask), v);
    }

    // phase 4: chunk of 8 sorted entries per thread (the first 256 threads), runs
    // summed in registers
    const uint32_t total = L.total;
    const uint32_t b0 = (uint32_t)tid * CHUNK;
    uint32_t mps[CHUNK];
    float mw[CHUNK], mg[CHUNK], md[CHUNK];
    int nmine = 0;
    if (tid < BLOCK && b0 < total) {
        nmine = min((int)(total - b0), CHUNK);
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) {
            if (j < nmine) {
                const float4 v = L.u.e.ent[stage_pos(b0 + j)];
                mps[j] = __float_as_uint(v.x);
                mw[j] = v.y;
                mg[j] = v.z;
                md[j] = v.w;
            }
        }
    }
    __syncthreads();  // the staging area is reused for the partials and totals below
    // The chunk's runs: summed with entry_acc; if a run's totals are not all
    // finite (a non-finite entry), the chunk is summed again with entry_sums, which
    // drops the non-finite sums of each entry, and its partials are rewritten.
    const float X0 = (float)col0 + 0.5f, Y0 = (float)row0 + 0.5f;  // exact: integers and halves
    auto sum_chunk = [&](bool checked) {
        float run[NSUM];
#pragma unroll
        for (int a = 0; a < NSUM; ++a)
            run[a] = 0.0f;
        int cur = (int)(mps[0] >> 8);
        SiteRec Rc = table_rec(L.T, cur);
        bool first = true, finite = true;
        auto close_run = [&](float *dst, int stride) {
            float all = run[0];
#pragma unroll
            for (int a = 0; a < NSUM; ++a) {
                if (a > 0)
                    all += run[a];
                dst[a * stride] = run[a];
                run[a] = 0.0f;
            }
            finite &= finitef(all);
        };
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) {
            if (j < nmine) {
                const int sl = (int)(mps[j] >> 8);
                if (sl != cur) {
                    // close the run of `cur`: the chunk's first run becomes its head
                    // partial; a later run is a whole bucket: its total is final
                    close_run(first ? &L.u.r.part[0][tid] : &L.u.r.fin[0][cur], first ? BLOCK : TBL);
                    first = false;
                    cur = sl;
                    Rc = table_rec(L.T, cur);
                }
                const int q = (int)(mps[j] & 0xFFu);
                const float Xp = (float)(q & (TILE - 1)) + X0, Yp = (float)(q / TILE) + Y0;
                if (checked) {
                    float v[NSUM];
                    entry_sums(Rc, Xp, Yp, mw[j], mg[j], md[j], L.g[q], v);
#pragma unroll
                    for (int a = 0; a < NSUM; ++a)
                        run[a] += v[a];
                } else {
                    entry_acc(Rc, Xp, Yp, mw[j], mg[j], md[j], L.g[q], run);
                }
            }
        }
        // the last run: head if it is also the first, else tail
        close_run(&L.u.r.part[first ? 0 : NSUM][tid], BLOCK);
        return finite;
    };
    if (nmine > 0 && !sum_chunk(false))
        sum_chunk(true);
    __syncthreads();

    // phase 5: eight lanes per occupied slot (the compacted list) add up the chunk
    // partials of its bucket -- lane r takes every eighth chunk from the r-th, then
    // the eight sums meet by lane exchanges -- and the first turns the totals into
    // the site's 11 gradient contributions.  (A site in every list of the tile
    // spans 256 entries, 32 chunks; one thread walking them all held the whole
    // workgroup at the next barrier.)
    {
        constexpr int GRP = 8;
        const int r = tid & (GRP - 1);
        for (int j = tid / GRP; j < (int)L.n_occ; j += PAIR_THREADS / GRP) {
            const int sl = L.occ[j];
            const uint32_t c = L.cnt[sl];
            const uint32_t b = L.off[sl], e = b + c - 1;
            const uint32_t t0c = b / CHUNK, t1c = e / CHUNK;
            const uint32_t end0 = min(t0c * CHUNK + CHUNK, total) - 1;
            const bool starts_chunk = (b == t0c * CHUNK);
            float v[NSUM];
#pragma unroll
            for (int a = 0; a < NSUM; ++a)
                v[a] = 0.0f;
            if (t0c != t1c || starts_chunk || e == end0) {
                if (r == 0) {
                    const int h0 = starts_chunk ? 0 : NSUM;
#pragma unroll
                    for (int a = 0; a < NSUM; ++a)
                        v[a] = L.u.r.part[h0 + a][t0c];
                }
                for (uint32_t tc = t0c + 1 + r; tc <= t1c; tc += GRP) {
#pragma unroll
                    for (int a = 0; a < NSUM; ++a)
                        v[a] += L.u.r.part[a][tc];
                }
            } else if (r == 0) {  // a middle run: its total is already in place
#pragma unroll
                for (int a = 0; a < NSUM; ++a)
                    v[a] = L.u.r.fin[a][sl];
            }
#pragma unroll
            for (int a = 0; a < NSUM; ++a)
                v[a] = group8_sum(v[a]);
            if (r == 0) {
                float acc[SAD_NACC];
                site_grads(table_rec(L.T, sl), s, v, acc);
#pragma unroll
                for (int a = 0; a < SAD_NACC; ++a)
                    L.u.r.fin[a][sl] = acc[a];
            }
        }
    }
    __syncthreads();

    // phase 6: cooperative flush -- consecutive lanes take consecutive accumulators
    // of one site, so the lanes of an atomic instruction share the site's 64-byte
    // gradient record instead of touching one cache line each
    const int n_items = (int)L.n_occ * SAD_NACC;
    for (int i = tid; i < n_items; i += PAIR_THREADS) {
        const int j = i / SAD_NACC, a = i - j * SAD_NACC;
        const int sl = L.occ[j];
        const float v = L.u.r.fin[a][sl];
        if (v != 0.0f)
            unsafeAtomicAdd(grad_at<GL>(grad, L.T.key[sl], a), v);
    }
}

// ---------------------------------------------------------------------------
// Budget-control statistics (summary, B.5: splitting is decided from a site's
// coverage, its remaining error and the spread of that error).  For each site, over the
// pixels x whose list holds it, with w its softmax weight at x, e = ||c(x) - t(x)||^2
// and delta = x - p (the site position, so the moments stay well conditioned):
//   [0] sum w   [1] sum w e   [2] sum w e dx   [3] sum w e dy
//   [4] sum w e dx^2   [5] sum w e dx dy   [6] sum w e dy^2   [7] unused
// accumulated (+=) into float [n][SAD_STAT_LD].  Entries of table sites add into
// a per-tile LDS accumulator (LDS float atomics: the kernel runs every few dozen
// iterations, so the simplest reduction that keeps global traffic per site per
// tile will do), flushed with one global atomic per site and statistic;
// entries whose site found no table slot go through the per-wave cooperative
// path.
constexpr int NSTAT = 7;

__global__ __launch_bounds__(BLOCK) void k_densify_stats(SiteSrc src, uint32_t n_slots,
                                                         const uint4 *__restrict__ cand,
                                                         const float *__restrict__ target, int W, int H,
                                                         float *__restrict__ stats, float s, MapGrid mg, int tiles_x,
                                                         int nb)
{
    __shared__ TileTable T;
    __shared__ float acc_t[NSTAT][TBL];
    __shared__ float stage[BLOCK / 64][64 * NSTAT + 64];
    const int tid = threadIdx.x, lane = tid & 63;
    int col, row;
    tile_pixel(nb, tiles_x, col, row);
    const bool inside = col < W && row < H;
    const long p = (long)row * W + col;
    uint32_t ids[K];
    int slot[K];
    load_ids(cand, mg.entry(p, col, row), inside, ids, col & 1, (col >> 1) & 1, (col >> 2) & 1);
    static_assert(TBL == BLOCK, "one accumulator column per thread");
#pragma unroll
    for (int a = 0; a < NSTAT; ++a)
        acc_t[a][tid] = 0.0f;  // complete at the table build's barriers
    build_tile_table<SEL_REC>(T, src, n_slots, ids, slot);
    const float X = (float)col + 0.5f, Y = (float)row + 0.5f;
    PixelBlend B;
    float err = 0.0f, iZ = 0.0f;
    bool any = false;
    if (inside) {
        blend_pixel<SEL_REC>(T, src, ids, slot, X, Y, s, B);
        const float r0 = B.chat0 - target[3 * p], r1 = B.chat1 - target[3 * p + 1], r2 = B.chat2 - target[3 * p + 2];
        err = r0 * r0 + r1 * r1 + r2 * r2;
        any = B.any;
        iZ = any ? hw_rcp(B.Z) : 0.0f;
    }
    float *vals = stage[tid >> 6];
    uint32_t *vid = reinterpret_cast<uint32_t *>(vals + 64 * NSTAT);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const bool has = any && B.use[k] && B.e[k] > 0.0f;
        if (!__any(has))
            continue;
        float acc[NSTAT];
#pragma unroll
        for (int a = 0; a < NSTAT; ++a)
            acc[a] = 0.0f;
        if (has) {
            const SiteRec R = fetch_rec<SEL_REC>(T, src, ids[k], slot[k]);
            const float w = B.e[k] * iZ, we = w * err;
            const float dx = X - R.v[R_PX], dy = Y - R.v[R_PY];
            acc[0] = w;
            acc[1] = we;
            acc[2] = we * dx;
            acc[3] = we * dy;
            acc[4] = we * dx * dx;
            acc[5] = we * dx * dy;
            acc[6] = we * dy * dy;
#pragma unroll
            for (int a = 0; a < NSTAT; ++a)
                acc[a] = finitef(acc[a]) ? acc[a] : 0.0f;
            if (slot[k] >= 0) {
#pragma unroll
                for (int a = 0; a < NSTAT; ++a)
                    if (acc[a] != 0.0f)
                        atomicAdd(&acc_t[a][slot[k]], acc[a]);
            }
        }
        const bool spilled = has && slot[k] < 0;
        if (!__any(spilled))
            continue;
#pragma unroll
        for (int a = 0; a < NSTAT; ++a)
            vals[lane * NSTAT + a] = spilled ? acc[a] : 0.0f;
        vid[lane] = spilled ? ids[k] : NONE;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int i = lane; i < 64 * NSTAT; i += 64) {
            const int e = i / NSTAT, a = i - e * NSTAT;
            const uint32_t c = vid[e];
            const float v = vals[i];
            if (c != NONE && v != 0.0f)
                unsafeAtomicAdd(&stats[(size_t)c * SAD_STAT_LD + a], v);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
    // one global atomic per site and statistic for the tile: consecutive lanes take
    // consecutive statistics of one site
    for (int i = tid; i < TBL * NSTAT; i += BLOCK) {
        const int sl = i / NSTAT, a = i - sl * NSTAT;
        const uint32_t c = T.key[sl];
        const float v = acc_t[a][sl];
        if (c != NONE && v != 0.0f)
            unsafeAtomicAdd(&stats[(size_t)c * SAD_STAT_LD + a], v);
    }
}

// ---------------------------------------------------------------------------
// 16-byte evaluation format (summary, Appendix B.2 "Packed storage for
// evaluation"; press article, section 5: 15-bit fixed-point coordinates, colour in
// 11/11/10 bits, 16 bits each for log tau and r with per-image min/scale, a 16-bit
// direction angle, float16 anisotropy) and the random-access query.
//   w0 = qx | qy << 15 | inactive << 31      w1 = qR | qG << 11 | qB << 22
//   w2 = q_logtau | q_r << 16                w3 = q_angle | f16(a) << 16
// Codes are rint (nearest even) of one float32 product (log tau and r: of
// (v - min) * inv), clamped to [0, qmax] with NaN -> 0.  The direction is an axis:
// the angle of atan2(dy, dx) folded into [0, pi), coded in float64 (float32 atan2
// implementations differ by an ulp, which would move codes near ties).
constexpr int EV_QPOS = 32767, EV_QRG = 2047, EV_QB = 1023, EV_Q16 = 65535;

__device__ __forceinline__ uint32_t ev_key(float v)  // order-preserving bits
{
    uint32_t u = __float_as_uint(v + 0.0f);
    return u ^ ((u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float ev_unkey(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
__device__ __forceinline__ uint32_t ev_quant(float t, float qmax)
{
    t = rintf(t);
    t = (t >= 0.0f) ? t : 0.0f;  // NaN -> 0
    return (uint32_t)fminf(t, qmax);
}

// keys: [lt_min, lt_max, r_min, r_max] as order-preserving bits (min starts at
// all ones, max at 0); a min still all ones afterwards means no finite value.
__global__ __launch_bounds__(64) void k_eval_range_init(uint32_t *__restrict__ keys)
{
    if (threadIdx.x < 4)
        keys[threadIdx.x] = (threadIdx.x & 1) ? 0u : 0xFFFFFFFFu;
}

__global__ __launch_bounds__(256) void k_eval_range(const float *__restrict__ S, int n_slots, int stride,
                                                    uint32_t *__restrict__ keys)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    uint32_t kmin[2] = {0xFFFFFFFFu, 0xFFFFFFFFu}, kmax[2] = {0u, 0u};
    if (i < n_slots && !(S[i] < 0.0f)) {
        const float v[2] = {S[PLT * (long)stride + i], S[PR * (long)stride + i]};
#pragma unroll
        for (int f = 0; f < 2; ++f)
            if (finitef(v[f])) {
                kmin[f] = ev_key(v[f]);
                kmax[f] = kmin[f];
            }
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            kmin[f] = min(kmin[f], (uint32_t)__shfl_xor((int)kmin[f], o));
            kmax[f] = max(kmax[f], (uint32_t)__shfl_xor((int)kmax[f], o));
        }
    }
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            if (kmin[f] != 0xFFFFFFFFu)
                atomicMin(keys + 2 * f, kmin[f]);
            if (kmax[f] != 0u)
                atomicMax(keys + 2 * f + 1, kmax[f]);
        }
    }
}

__device__ __forceinline__ void ev_range(const uint32_t *keys, int f, float &m, float &M)
{
    if (keys[2 * f] == 0xFFFFFFFFu) {
        m = M = 0.0f;
    } else {
        m = ev_unkey(keys[2 * f]);
        M = ev_unkey(keys[2 * f + 1]);
    }
}

__global__ __launch_bounds__(256) void k_eval_encode(const float *__restrict__ S, int n_slots, int stride, float sxe,
                                                     float sye, const uint32_t *__restrict__ keys,
                                                     uint4 *__restrict__ words)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n_slots)
        return;
    const long st = stride;
    const float x = S[i];
    if (x < 0.0f) {
        words[i] = make_uint4(0x80000000u, 0u, 0u, 0u);
        return;
    }
    float lm, lM, rm, rM;
    ev_range(keys, 0, lm, lM);
    ev_range(keys, 1, rm, rM);
    const float linv = lM > lm ? (float)EV_Q16 / (lM - lm) : 0.0f;
    const float rinv = rM > rm ? (float)EV_Q16 / (rM - rm) : 0.0f;
    const uint32_t qx = ev_quant(x * sxe, (float)EV_QPOS), qy = ev_quant(S[st + i] * sye, (float)EV_QPOS);
    const uint32_t qr = ev_quant(S[PCR * st + i] * (float)EV_QRG, (float)EV_QRG);
    const uint32_t qg = ev_quant(S[PCG * st + i] * (float)EV_QRG, (float)EV_QRG);
    const uint32_t qb = ev_quant(S[PCB * st + i] * (float)EV_QB, (float)EV_QB);
    const uint32_t ql = ev_quant((S[PLT * st + i] - lm) * linv, (float)EV_Q16);
    const uint32_t qd = ev_quant((S[PR * st + i] - rm) * rinv, (float)EV_Q16);
    const double dx = S[PDX * st + i], dy = S[PDY * st + i];
    uint32_t qa = 0;
    if (!(__dadd_rn(__dmul_rn(dx, dx), __dmul_rn(dy, dy)) < 1e-30)) {
        double th = atan2(dy, dx);
        if (th < 0.0)
            th += 3.141592653589793;
        const double t = rint(th * (65536.0 / 3.141592653589793));
        qa = __builtin_isfinite(t) ? (uint32_t)(long long)t & 0xFFFFu : 0u;
    }
    words[i] = make_uint4(qx | (qy << 15), qr | (qg << 11) | (qb << 22), ql | (qd << 16),
                          qa | (f16_bits(S[PA * st + i]) << 16));
}

// keys -> header [lt_min, lt_step, r_min, r_step], step = (max - min) / 65535.
__global__ __launch_bounds__(64) void k_eval_header(uint32_t *__restrict__ keys)
{
    if (threadIdx.x != 0)
        return;
    float lm, lM, rm, rM;
    ev_range(keys, 0, lm, lM);
    ev_range(keys, 1, rm, rM);
    float *h = reinterpret_cast<float *>(keys);
    h[0] = lm;
    h[1] = (lM - lm) / (float)EV_Q16;
    h[2] = rm;
    h[3] = (rM - rm) / (float)EV_Q16;
}

// Decoded site, float32, each operation rounded on its own (no contraction) so
// that every value is reproducible: position, colour, log tau, r, angle, a.
struct EvSite {
    float x, y, lt, r, c0, c1, c2, th, a;
    bool active;
};

__device__ __forceinline__ EvSite ev_decode(uint4 w, const float4 &hd, float dxe, float dye)
{
#pragma clang fp contract(off)  // log tau and r: a rounded product, then a rounded sum
    EvSite e;
    e.active = (w.x >> 31) == 0u;
    e.x = (float)(w.x & 0x7FFFu) * dxe;
    e.y = (float)((w.x >> 15) & 0x7FFFu) * dye;
    e.c0 = (float)(w.y & 0x7FFu) * (1.0f / (float)EV_QRG);
    e.c1 = (float)((w.y >> 11) & 0x7FFu) * (1.0f / (float)EV_QRG);
    e.c2 = (float)(w.y >> 22) * (1.0f / (float)EV_QB);
    const float qlt = (float)(w.z & 0xFFFFu) * hd.y, qr = (float)(w.z >> 16) * hd.w;
    e.lt = hd.x + qlt;
    e.r = hd.z + qr;
    e.th = (float)(w.w & 0xFFFFu) * (float)(3.141592653589793 / 65536.0);
    e.a = half_hi(w.w);
    return e;
}

__global__ __launch_bounds__(256) void k_eval_decode(const uint4 *__restrict__ words, const float4 *__restrict__ hdr,
                                                     int n_slots, float dxe, float dye, float *__restrict__ S,
                                                     int stride)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n_slots)
        return;
    const long st = stride;
    const EvSite e = ev_decode(words[i], hdr[0], dxe, dye);
    float v[SAD_NPARAM] = {-1.0f, -1.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (e.active) {
        float sn, cs;
        sincosf(e.th, &sn, &cs);
        v[PX] = e.x;
        v[PY] = e.y;
        v[PLT] = e.lt;
        v[PR] = e.r;
        v[PCR] = e.c0;
        v[PCG] = e.c1;
        v[PCB] = e.c2;
        v[PDX] = cs;
        v[PDY] = sn;
        v[PA] = e.a;
    }
#pragma unroll
    for (int j = 0; j < SAD_NPARAM; ++j)
        S[j * st + i] = v[j];
}

// Random-access query: point i reads the list of the map entry of the pixel that
// holds it (coordinates clamped into the image) and blends its sites, decoded
// from the evaluation words, at the point itself (the render's score and
// max-subtracted softmax).  A non-finite coordinate returns 0.
__global__ __launch_bounds__(256) void k_eval_query(const uint4 *__restrict__ words, const float4 *__restrict__ hdr,
                                                    uint32_t n_slots, const uint4 *__restrict__ cand, int W, int H,
                                                    MapGrid mg, const float2 *__restrict__ pts, long n_pts,
                                                    float *__restrict__ out, float s, float dxe, float dye)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_pts)
        return;
    const float2 P = pts[i];
    float o0 = 0.0f, o1 = 0.0f, o2 = 0.0f;
    if (finitef(P.x) && finitef(P.y)) {
        const int col = (int)floorf(fminf(fmaxf(P.x, 0.0f), (float)(W - 1)));
        const int row = (int)floorf(fminf(fmaxf(P.y, 0.0f), (float)(H - 1)));
        const long q = mg.entry((long)row * W + col, col, row);
        const uint4 la = cand[2 * q], lb = cand[2 * q + 1];
        const uint32_t ids[K] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        const float4 hd = hdr[0];
        float l[K], c0[K], c1[K], c2[K];
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            l[k] = -__builtin_huge_valf();
            c0[k] = c1[k] = c2[k] = 0.0f;
            if (ids[k] >= n_slots)
                continue;
            const EvSite e = ev_decode(words[ids[k]], hd, dxe, dye);
            if (!e.active)
                continue;
            float sn, cs;
            sincosf(e.th, &sn, &cs);
            const float ex = P.x - e.x, ey = P.y - e.y;
            const float al = fmaf(cs, ex, sn * ey), be = fmaf(cs, ey, -(sn * ex));
            const float E = __expf(e.a), iE = __expf(-e.a);
            const float d = fmaf(s, hw_sqrt(fmaf(E * al, al, iE * be * be)), -(s * e.r));
            const float lk = -__expf(e.lt) * d;
            if (!finitef(lk))
                continue;
            l[k] = lk;
            c0[k] = e.c0;
            c1[k] = e.c1;
            c2[k] = e.c2;
            mx = fmaxf(mx, lk);
        }
        if (mx > -__builtin_huge_valf()) {
            float Z = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float ek = l[k] > -__builtin_huge_valf() ? __expf(l[k] - mx) : 0.0f;
                Z += ek;
                o0 = fmaf(ek, c0[k], o0);
                o1 = fmaf(ek, c1[k], o1);
                o2 = fmaf(ek, c2[k], o2);
            }
            const float iZ = hw_rcp(Z);  // Z >= 1
            o0 *= iZ;
            o1 *= iZ;
            o2 *= iZ;
        }
    }
    out[3 * i] = o0;
    out[3 * i + 1] = o1;
    out[3 * i + 2] = o2;
}

// ---------------------------------------------------------------------------
// Adam (Kingma & Ba 2015) on the ten site parameters, gradients divided by the
// pixel count (summary, B.4), gradient planes 0..9 zeroed in the same pass.
struct AdamArgs {
    float lr[SAD_NPARAM];
    float b1, b2, eps, ibc1, ibc2, inv_p, W, H;  // ibc = 1 / (1 - beta^step)
    float qsx, qsy;                              // 4096 / W, 4096 / H: the screen's cells
};

template <int GL>
__global__ __launch_bounds__(256) void k_adam(float *__restrict__ S, float *__restrict__ M, float *__restrict__ V,
                                              float *__restrict__ G, float4 *__restrict__ rec,
                                              uint4 *__restrict__ packed, uint32_t *__restrict__ scr, int n_slots,
                                              int stride, AdamArgs A)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n_slots)
        return;
    const long st = stride;
    float gv[SAD_NPARAM];
    if constexpr (GL == GL_REC) {
        float4 *gr = reinterpret_cast<float4 *>(G + (long)i * SAD_GRAD_LD);
        const float4 ga = gr[0], gb = gr[1], gc = gr[2];
        gv[0] = ga.x; gv[1] = ga.y; gv[2] = ga.z; gv[3] = ga.w;
        gv[4] = gb.x; gv[5] = gb.y; gv[6] = gb.z; gv[7] = gb.w;
        gv[8] = gc.x; gv[9] = gc.y;
    } else {
#pragma unroll
        for (int j = 0; j < SAD_NPARAM; ++j)
            gv[j] = G[j * st + i];
    }
    // every load first (parameters, then moments), the updates in registers, then
    // the stores and the derived record: one memory round trip per slot instead
    // of one per parameter
    float po[SAD_NPARAM];
#pragma unroll
    for (int j = 0; j < SAD_NPARAM; ++j)
        po[j] = S[j * st + i];
    if constexpr (GL == GL_REC) {
        float4 *gr = reinterpret_cast<float4 *>(G + (long)i * SAD_GRAD_LD);
        gr[0] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        gr[1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        reinterpret_cast<float2 *>(gr + 2)[0] = make_float2(0.0f, 0.0f);
    } else {
#pragma unroll
        for (int j = 0; j < SAD_NPARAM; ++j)
            G[j * st + i] = 0.0f;
    }
    const bool active = !(po[PX] < 0.0f);
    if (active) {
        float mo[SAD_NPARAM], vo[SAD_NPARAM];
#pragma unroll
        for (int j = 0; j < SAD_NPARAM; ++j) {
            mo[j] = M[j * st + i];
            vo[j] = V[j * st + i];
        }
#pragma unroll
        for (int j = 0; j < SAD_NPARAM; ++j) {
            float g = gv[j] * A.inv_p;
            if (!finitef(g))
                g = 0.0f;
            const float m = A.b1 * mo[j] + (1.0f - A.b1) * g;
            const float v = A.b2 * vo[j] + (1.0f - A.b2) * g * g;
            mo[j] = m;
            vo[j] = v;
            po[j] = po[j] - A.lr[j] * (m * A.ibc1) * hw_rcp(hw_sqrt(v * A.ibc2) + A.eps);
        }
        po[PX] = po[PX] < 0.0f ? 0.0f : (po[PX] > A.W ? A.W : po[PX]);
        po[PY] = po[PY] < 0.0f ? 0.0f : (po[PY] > A.H ? A.H : po[PY]);
#pragma unroll
        for (int j = 0; j < SAD_NPARAM; ++j) {
            M[j * st + i] = mo[j];
            V[j * st + i] = vo[j];
            S[j * st + i] = po[j];
        }
    }
    if (rec) {
        float4 o[RLD4];
        make_record_v(po, o);
#pragma unroll
        for (int j = 0; j < RLD4; ++j)
            rec[RLD4 * (size_t)i + j] = o[j];
    }
    if (packed)
        packed[i] = pack_site_v(po);
    if (scr)
        scr[i] = screen_word(po[PX], po[PY], po[PR], po[PA], A.qsx, A.qsy);
}

// ---------------------------------------------------------------------------
// Host helpers.
inline int check_image(int W, int H)
{
    if (W < 0 || H < 0 || W > SAD_MAX_DIM || H > SAD_MAX_DIM)
        return SAD_ERR_ARG;
    return SAD_OK;
}

inline int check_sites(int n_slots, int stride)
{
    if (n_slots < 0 || stride < 1 || n_slots > stride)
        return SAD_ERR_ARG;
    return SAD_OK;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline float scale_of(int W, int H) { return 1.0f / (float)(W > H ? W : H); }

// The map grid of a W x H image with cells of `cell` pixels (W, H > 0); false if
// the cell size is out of range.
inline bool map_grid(int W, int H, int cell, MapGrid &mg, int &Wm, int &Hm)
{
    if (cell < 1 || cell > SAD_MAX_DIM)
        return false;
    Wm = (W + cell - 1) / cell;
    Hm = (H + cell - 1) / cell;
    mg.c = cell;
    mg.Wm = Wm;
    mg.sx = (float)W / (float)Wm;
    mg.sy = (float)H / (float)Hm;
    return true;
}

struct TileGrid {
    int tiles_x, nb;
};

inline TileGrid tile_grid(int W, int H, int tw = TILE)
{
    TileGrid g;
    g.tiles_x = (W + tw - 1) / tw;
    g.nb = g.tiles_x * ((H + tw - 1) / tw);
    return g;
}

// A launch of fewer 16x16 tiles than this leaves CUs idle (256 CUs, several
// workgroups each): the table-free pass then runs on 8x8 tiles.
constexpr int SMALL_MAP_TILES = 1024;

inline int launched()
{
    return hipGetLastError() == hipSuccess ? SAD_OK : SAD_ERR_DEVICE;
}

inline bool valid_fmt(int f) { return f == SEL_REC || f == SEL_PACKED; }

struct PropArgs {
    SiteSrc src;
    Screen sc;
    uint32_t n;
    const uint4 *ci;
    uint4 *co;
    int Wm, Hm, cell, jump;
    uint32_t seed_h;
    int n_inject;
    float s, sx, sy;
};

// Per-pixel maps: jumps up to 4 run the tile table over the tile and its ring
// of jump-wide strips, whose per-pixel bitmap skips the entries the pixel has
// scored already (at 4096x4096, 1M sites, after an edit: jump 2 0.94 vs 1.34 ms
// in the five-region table, jump 4 1.12 vs 1.35 ms; at jump 8, 1.69 vs 1.49, it
// loses).  Larger jumps run the five-region table (k_propagate_wide; a sparse
// 2048-key hash from jump 16 on), which at that size with 8 injected IDs beats
// fetching every candidate's record (17.4 vs 20.8 ms for the 12-pass refresh;
// without injection 14.0 vs 13.9 ms).  On a downscaled map
// (cell > 1) a 16x16 tile spans c^2 times the pixels and its lists name more
// sites than a table holds: every pass is table-free there, on 8x8 tiles when
// 16x16 ones would leave CUs idle.
template <int FMT>
void launch_propagate(const PropArgs &A, hipStream_t hs)
{
    const TileGrid g = tile_grid(A.Wm, A.Hm);
    if (A.cell > 1 && g.nb < SMALL_MAP_TILES) {
        const TileGrid g8 = tile_grid(A.Wm, A.Hm, 8);
        hipLaunchKernelGGL((k_propagate_direct<8, FMT>), dim3(g8.nb), dim3(64), 0, hs, A.src, A.sc, A.n, A.ci, A.co, A.Wm,
                           A.Hm, A.jump, A.seed_h, A.n_inject, A.s, A.sx, A.sy, g8.tiles_x, g8.nb);
    } else if (A.cell == 1 && A.jump == 1) {
        hipLaunchKernelGGL((k_propagate<1, 256, FMT>), dim3(g.nb), dim3(BLOCK), 0, hs, A.src, A.sc, A.n, A.ci, A.co,
                           A.Wm, A.Hm, A.jump, A.seed_h, A.n_inject, A.s, A.sx, A.sy, g.tiles_x, g.nb);
    } else if (A.cell == 1 && A.jump == 2) {
        hipLaunchKernelGGL((k_propagate<2, 256, FMT>), dim3(g.nb), dim3(BLOCK), 0, hs, A.src, A.sc, A.n, A.ci, A.co,
                           A.Wm, A.Hm, A.jump, A.seed_h, A.n_inject, A.s, A.sx, A.sy, g.tiles_x, g.nb);
    } else if (A.cell == 1 && A.jump <= 4) {
        hipLaunchKernelGGL((k_propagate<4, 256, FMT>), dim3(g.nb), dim3(BLOCK), 0, hs, A.src, A.sc, A.n, A.ci, A.co,
                           A.Wm, A.Hm, A.jump, A.seed_h, A.n_inject, A.s, A.sx, A.sy, g.tiles_x, g.nb);
    } else if (A.cell == 1) {
        if (A.jump >= 16)
            hipLaunchKernelGGL((k_propagate_wide<FMT, WKT_SPARSE>), dim3(g.nb), dim3(BLOCK), 0, hs, A.src, A.sc, A.n,
                               A.ci, A.co, A.Wm, A.Hm, A.jump, A.seed_h, A.n_inject, A.s, g.tiles_x, g.nb);
        else
            hipLaunchKernelGGL((k_propagate_wide<FMT, WTB>), dim3(g.nb), dim3(BLOCK), 0, hs, A.src, A.sc, A.n, A.ci,
                               A.co, A.Wm, A.Hm, A.jump, A.seed_h, A.n_inject, A.s, g.tiles_x, g.nb);
    } else {
        hipLaunchKernelGGL((k_propagate_direct<TILE, FMT>), dim3(g.nb), dim3(BLOCK), 0, hs, A.src, A.sc, A.n, A.ci,
                           A.co,
                           A.Wm, A.Hm, A.jump, A.seed_h, A.n_inject, A.s, A.sx, A.sy, g.tiles_x, g.nb);
    }
}

uint32_t host_pcg_hash(uint32_t v)
{
    const uint32_t state = v * 747796405u + 2891336453u;
    const uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
    return (word >> 22u) ^ word;
}

inline SiteSrc src_of(const float *rec) { return SiteSrc{(const float4 *)rec, nullptr, 0}; }

// The screen of a W x H image (scr may be NULL: no screening).
inline Screen screen_of(const uint32_t *scr, int W, int H)
{
    return Screen{scr, (float)W / SCR_Q, (float)H / SCR_Q, (float)(W > H ? W : H)};
}
inline SiteSrc src_planes(const float *sites, int stride) { return SiteSrc{nullptr, sites, (long)stride}; }

// One propagation pass from any site source (fmt: SEL_REC, SEL_PACKED or SEL_SOA);
// `site_ptr` is the pointer the source reads, for the NULL check.
int propagate_pass(SiteSrc src, const void *site_ptr, int fmt, const uint32_t *scr, int n_slots,
                   const uint32_t *cand_in, uint32_t *cand_out, int W, int H, int cell, int jump, uint32_t pass_index,
                   uint32_t seed, int n_inject, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || jump < 1 || jump > 0xFFFF || n_inject < 0 || n_inject > SAD_MAX_INJECT || cell < 1)
        return SAD_ERR_ARG;
    if (W == 0 || H == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!site_ptr && n_slots > 0) || !cand_in || !cand_out)
        return SAD_ERR_ARG;
    const size_t bytes = (size_t)Wm * Hm * K * sizeof(uint32_t);
    const uintptr_t a0 = (uintptr_t)cand_in, a1 = (uintptr_t)cand_out;
    if (a0 < a1 + bytes && a1 < a0 + bytes)
        return SAD_ERR_ARG;
    if (!aligned16(cand_in) || !aligned16(cand_out) || (fmt != SEL_SOA && !aligned16(site_ptr)) ||
        ((uintptr_t)scr & 3u))
        return SAD_ERR_ALIGN;
    const uint32_t pw = ((uint32_t)jump << 16) | (pass_index & 0xFFFFu);
    const uint32_t seed_h = host_pcg_hash(host_pcg_hash(seed) ^ pw);
    // the screen bounds float32 scores; selection from the packed buffer ranks
    // float16-rounded sites, for which it does not hold
    const PropArgs A{src, screen_of(n_slots > 0 && fmt == SEL_REC ? scr : nullptr, W, H), (uint32_t)n_slots, (const uint4 *)cand_in, (uint4 *)cand_out, Wm, Hm,
                     cell, jump, seed_h, n_inject, scale_of(W, H), mg.sx, mg.sy};
    if (fmt == SEL_PACKED)
        launch_propagate<SEL_PACKED>(A, (hipStream_t)stream);
    else if (fmt == SEL_SOA)
        launch_propagate<SEL_SOA>(A, (hipStream_t)stream);
    else
        launch_propagate<SEL_REC>(A, (hipStream_t)stream);
    return launched();
}

int render_fwd_any(SiteSrc src, const void *site_ptr, int fmt, int n_slots, const uint32_t *cand, int W, int H,
                   int cell, float *out_rgb, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || cell < 1)
        return SAD_ERR_ARG;
    if (W == 0 || H == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!site_ptr && n_slots > 0) || !cand || !out_rgb)
        return SAD_ERR_ARG;
    if (!aligned16(cand) || (fmt != SEL_SOA && !aligned16(site_ptr)))
        return SAD_ERR_ALIGN;
    const TileGrid g = tile_grid(W, H);
    if (fmt == SEL_SOA)
        hipLaunchKernelGGL(k_render_fwd<SEL_SOA>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (const uint4 *)cand, W, H, out_rgb, scale_of(W, H), mg, g.tiles_x, g.nb);
    else
        hipLaunchKernelGGL(k_render_fwd<SEL_REC>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (const uint4 *)cand, W, H, out_rgb, scale_of(W, H), mg, g.tiles_x, g.nb);
    return launched();
}

int adam_any(float *sites, float *m, float *v, float *grad, int gl, float *rec, uint32_t *packed, uint32_t *scr,
             int n_slots, int stride, int step, int n_pixels, const sad_adam_cfg *cfg, void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)))
        return rc;
    if (!sites || !m || !v || !grad || !cfg || step < 1 || n_pixels < 1)
        return SAD_ERR_ARG;
    if (!(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f && cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f && cfg->eps >= 0.0f))
        return SAD_ERR_ARG;
    if (!(cfg->x_max > 0.0f && cfg->y_max > 0.0f && cfg->x_max <= (float)SAD_MAX_DIM &&
          cfg->y_max <= (float)SAD_MAX_DIM))
        return SAD_ERR_ARG;
    if ((gl == GL_REC && !aligned16(grad)) || !aligned16(rec) || !aligned16(packed) || ((uintptr_t)scr & 3u))
        return SAD_ERR_ALIGN;
    if (n_slots == 0)
        return SAD_OK;
    AdamArgs A;
    for (int j = 0; j < SAD_NPARAM; ++j)
        A.lr[j] = cfg->lr[j];
    A.b1 = cfg->beta1;
    A.b2 = cfg->beta2;
    A.eps = cfg->eps;
    A.ibc1 = (float)(1.0 / (1.0 - __builtin_pow((double)cfg->beta1, (double)step)));
    A.ibc2 = (float)(1.0 / (1.0 - __builtin_pow((double)cfg->beta2, (double)step)));
    A.inv_p = 1.0f / (float)n_pixels;
    A.W = cfg->x_max;
    A.H = cfg->y_max;
    A.qsx = SCR_Q / cfg->x_max;
    A.qsy = SCR_Q / cfg->y_max;
    if (gl == GL_PLANES)
        hipLaunchKernelGGL(k_adam<GL_PLANES>, dim3((n_slots + 255) / 256), dim3(256), 0, (hipStream_t)stream, sites,
                           m, v, grad, (float4 *)rec, (uint4 *)packed, scr, n_slots, stride, A);
    else
        hipLaunchKernelGGL(k_adam<GL_REC>, dim3((n_slots + 255) / 256), dim3(256), 0, (hipStream_t)stream, sites, m,
                           v, grad, (float4 *)rec, (uint4 *)packed, scr, n_slots, stride, A);
    return launched();
}

}  // namespace

extern "C" {

int sad_abi_version(void) { return SAD_ABI_VERSION; }

const char *sad_status_string(int status)
{
    switch (status) {
    case SAD_OK: return "ok";
    case SAD_ERR_ARG: return "invalid argument";
    case SAD_ERR_ALIGN: return "misaligned pointer";
    case SAD_ERR_DEVICE: return "HIP launch failed";
    case SAD_ERR_CAPACITY: return "capacity exceeded";
    case SAD_ERR_UNIMPLEMENTED: return "not implemented";
    default: return "unknown status";
    }
}

int sad_site_records(const float *sites, int n_slots, int stride, float *rec, void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)))
        return rc;
    if (n_slots == 0)
        return SAD_OK;
    if (!sites || !rec)
        return SAD_ERR_ARG;
    if (!aligned16(rec))
        return SAD_ERR_ALIGN;
    hipLaunchKernelGGL(k_site_records, dim3((n_slots + 255) / 256), dim3(256), 0, (hipStream_t)stream, sites, n_slots,
                       stride, (float4 *)rec);
    return launched();
}

int sad_pack_sites(const float *sites, int n_slots, int stride, uint32_t *packed, void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)))
        return rc;
    if (n_slots == 0)
        return SAD_OK;
    if (!sites || !packed)
        return SAD_ERR_ARG;
    if (!aligned16(packed))
        return SAD_ERR_ALIGN;
    hipLaunchKernelGGL(k_pack_sites, dim3((n_slots + 255) / 256), dim3(256), 0, (hipStream_t)stream, sites, n_slots,
                       stride, (uint4 *)packed);
    return launched();
}

int sad_topk_propagate(const float *sites, int n_slots, int stride, const uint32_t *cand_in, uint32_t *cand_out, int W,
                       int H, int jump, uint32_t pass_index, uint32_t seed, int n_inject, void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)))
        return rc;
    return propagate_pass(src_planes(sites, stride), sites, SEL_SOA, nullptr, n_slots, cand_in, cand_out, W, H, 1,
                          jump, pass_index, seed, n_inject, stream);
}

int sad_topk_propagate_rec(const float *rec, int sel_fmt, const uint32_t *scr, int n_slots, const uint32_t *cand_in,
                           uint32_t *cand_out, int W, int H, int cell, int jump, uint32_t pass_index, uint32_t seed,
                           int n_inject, void *stream)
{
    if (!valid_fmt(sel_fmt))
        return SAD_ERR_ARG;
    return propagate_pass(src_of(rec), rec, sel_fmt, scr, n_slots, cand_in, cand_out, W, H, cell, jump, pass_index,
                          seed, n_inject, stream);
}

int sad_site_screen(const float *sites, int n_slots, int stride, int W, int H, uint32_t *scr, void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)) || (rc = check_image(W, H)))
        return rc;
    if (W < 1 || H < 1)
        return SAD_ERR_ARG;
    if (n_slots == 0)
        return SAD_OK;
    if (!sites || !scr)
        return SAD_ERR_ARG;
    if ((uintptr_t)scr & 3u)
        return SAD_ERR_ALIGN;
    hipLaunchKernelGGL(k_site_screen, dim3((n_slots + 255) / 256), dim3(256), 0, (hipStream_t)stream, sites, n_slots,
                       stride, SCR_Q / (float)W, SCR_Q / (float)H, scr);
    return launched();
}

int sad_apply_seeds(uint32_t *cand, int W, int H, int cell, const uint32_t *seeds, long n_seeds, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (cell < 1 || n_seeds < 0 || n_seeds > 0x7FFFFFFFL)
        return SAD_ERR_ARG;
    if (W == 0 || H == 0 || n_seeds == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if (!cand || !seeds)
        return SAD_ERR_ARG;
    if (!aligned16(cand) || ((uintptr_t)seeds & 7u))
        return SAD_ERR_ALIGN;
    hipLaunchKernelGGL(k_apply_seeds, dim3((unsigned)((n_seeds + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       cand, (long)Wm * Hm, (const uint2 *)seeds, n_seeds);
    return launched();
}

int sad_jfa_seed(const float *rec, int sel_fmt, int n_slots, uint32_t *cand, int W, int H, int cell, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || cell < 1 || !valid_fmt(sel_fmt))
        return SAD_ERR_ARG;
    if (W == 0 || H == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!rec && n_slots > 0) || !cand)
        return SAD_ERR_ARG;
    if (!aligned16(cand) || !aligned16(rec))
        return SAD_ERR_ALIGN;
    const long P = (long)Wm * Hm;
    const hipStream_t hs = (hipStream_t)stream;
    const SiteSrc src = src_of(rec);
    hipLaunchKernelGGL(k_fill_map, dim3((unsigned)((2 * P + 255) / 256)), dim3(256), 0, hs, (uint4 *)cand, 2 * P);
    if (n_slots > 0)
        for (int r = 0; r < JFA_KEEP; ++r) {
            if (sel_fmt == SEL_PACKED)
                hipLaunchKernelGGL(k_jfa_seed_round<SEL_PACKED>, dim3((n_slots + 255) / 256), dim3(256), 0, hs, src,
                                   (uint32_t)n_slots, (unsigned long long *)cand, W, H, scale_of(W, H), mg, r);
            else
                hipLaunchKernelGGL(k_jfa_seed_round<SEL_REC>, dim3((n_slots + 255) / 256), dim3(256), 0, hs, src,
                                   (uint32_t)n_slots, (unsigned long long *)cand, W, H, scale_of(W, H), mg, r);
        }
    hipLaunchKernelGGL(k_jfa_seed_finish, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, hs, (uint4 *)cand, P);
    return launched();
}

int sad_jfa_pass(const float *rec, int sel_fmt, int n_slots, const uint32_t *cand_in, uint32_t *cand_out, int W, int H,
                 int cell, int step, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || step < 1 || step > 0xFFFF || cell < 1 || !valid_fmt(sel_fmt))
        return SAD_ERR_ARG;
    if (W == 0 || H == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!rec && n_slots > 0) || !cand_in || !cand_out)
        return SAD_ERR_ARG;
    const size_t bytes = (size_t)Wm * Hm * K * sizeof(uint32_t);
    const uintptr_t a0 = (uintptr_t)cand_in, a1 = (uintptr_t)cand_out;
    if (a0 < a1 + bytes && a1 < a0 + bytes)
        return SAD_ERR_ARG;
    if (!aligned16(cand_in) || !aligned16(cand_out) || !aligned16(rec))
        return SAD_ERR_ALIGN;
    const TileGrid g = tile_grid(Wm, Hm);
    const SiteSrc src = src_of(rec);
    // Steps up to 8 on per-pixel maps through the tile table.  At larger steps the
    // nine lists of a pixel's neighbours still name sites of seeds far apart, a
    // tile's regions name thousands of sites and the table only overflows
    // (4096x4096 after the edit of 10 % of 1M sites: step 512 1.67 vs 1.03 ms,
    // steps 16-256 even, steps 8 / 4 / 2 2.54 / 1.35 / 1.24 vs 2.92 / 2.12 /
    // 1.72 ms); on the downscaled grid a tile of cells names more sites than the
    // table holds.  Both are table-free there.
    const bool table = cell == 1 && step <= 8;
    if (table && sel_fmt == SEL_PACKED)
        hipLaunchKernelGGL(k_jfa_pass_table<SEL_PACKED>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (const uint4 *)cand_in, (uint4 *)cand_out, Wm, Hm, step, scale_of(W, H),
                           g.tiles_x, g.nb);
    else if (table)
        hipLaunchKernelGGL(k_jfa_pass_table<SEL_REC>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (const uint4 *)cand_in, (uint4 *)cand_out, Wm, Hm, step, scale_of(W, H),
                           g.tiles_x, g.nb);
    else if (sel_fmt == SEL_PACKED)
        hipLaunchKernelGGL(k_jfa_pass<SEL_PACKED>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (const uint4 *)cand_in, (uint4 *)cand_out, Wm, Hm, step, scale_of(W, H),
                           mg.sx, mg.sy, g.tiles_x, g.nb);
    else
        hipLaunchKernelGGL(k_jfa_pass<SEL_REC>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (const uint4 *)cand_in, (uint4 *)cand_out, Wm, Hm, step, scale_of(W, H),
                           mg.sx, mg.sy, g.tiles_x, g.nb);
    return launched();
}

int sad_topk_exact(const float *rec, int sel_fmt, int n_slots, uint32_t *cand_out, int W, int H, int cell, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || cell < 1 || !valid_fmt(sel_fmt))
        return SAD_ERR_ARG;
    if (W == 0 || H == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!rec && n_slots > 0) || !cand_out)
        return SAD_ERR_ARG;
    if (!aligned16(cand_out) || !aligned16(rec))
        return SAD_ERR_ALIGN;
    const TileGrid g = tile_grid(Wm, Hm);
    const SiteSrc src = src_of(rec);
    if (sel_fmt == SEL_PACKED)
        hipLaunchKernelGGL(k_topk_exact<SEL_PACKED>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (uint4 *)cand_out, Wm, Hm, scale_of(W, H), mg.sx, mg.sy, g.tiles_x,
                           g.nb);
    else
        hipLaunchKernelGGL(k_topk_exact<SEL_REC>, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, (uint4 *)cand_out, Wm, Hm, scale_of(W, H), mg.sx, mg.sy, g.tiles_x,
                           g.nb);
    return launched();
}

int sad_topk_exact_at(const float *rec, int sel_fmt, int n_slots, const uint32_t *entries, int n_entries, int W, int H,
                      int cell, uint32_t *out, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || n_entries < 0 || cell < 1 || !valid_fmt(sel_fmt))
        return SAD_ERR_ARG;
    if (W == 0 || H == 0 || n_entries == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!rec && n_slots > 0) || !entries || !out)
        return SAD_ERR_ARG;
    if (!aligned16(out) || !aligned16(rec) || ((uintptr_t)entries & 3u))
        return SAD_ERR_ALIGN;
    const unsigned nb = (unsigned)((n_entries + BLOCK - 1) / BLOCK);
    const SiteSrc src = src_of(rec);
    if (sel_fmt == SEL_PACKED)
        hipLaunchKernelGGL(k_topk_exact_at<SEL_PACKED>, dim3(nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, entries, n_entries, (uint4 *)out, Wm, Hm, scale_of(W, H), mg.sx, mg.sy);
    else
        hipLaunchKernelGGL(k_topk_exact_at<SEL_REC>, dim3(nb), dim3(BLOCK), 0, (hipStream_t)stream, src,
                           (uint32_t)n_slots, entries, n_entries, (uint4 *)out, Wm, Hm, scale_of(W, H), mg.sx, mg.sy);
    return launched();
}

int sad_render_fwd(const float *sites, int n_slots, int stride, const uint32_t *cand, int W, int H, float *out_rgb,
                   void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)))
        return rc;
    return render_fwd_any(src_planes(sites, stride), sites, SEL_SOA, n_slots, cand, W, H, 1, out_rgb, stream);
}

int sad_render_fwd_rec(const float *rec, int n_slots, const uint32_t *cand, int W, int H, int cell, float *out_rgb,
                       void *stream)
{
    return render_fwd_any(src_of(rec), rec, SEL_REC, n_slots, cand, W, H, cell, out_rgb, stream);
}

int sad_render_bwd(const float *sites, int n_slots, int stride, const uint32_t *cand, const float *target, int W,
                   int H, float *grad, float *loss_sum, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)) || (rc = check_sites(n_slots, stride)))
        return rc;
    if (W == 0 || H == 0)
        return SAD_OK;
    if ((!sites && n_slots > 0) || !cand || !target || (!grad && n_slots > 0))
        return SAD_ERR_ARG;
    if (!aligned16(cand) || ((uintptr_t)sites & 3u) || ((uintptr_t)grad & 3u))
        return SAD_ERR_ALIGN;
    MapGrid mg;
    int Wm, Hm;
    map_grid(W, H, 1, mg, Wm, Hm);
    const TileGrid g = tile_grid(W, H);
    hipLaunchKernelGGL((k_render_bwd<SEL_SOA, GL_PLANES>), dim3(g.nb), dim3(PAIR_THREADS), 0, (hipStream_t)stream,
                       src_planes(sites, stride), (uint32_t)n_slots, (const uint4 *)cand, target, W, H,
                       GradOut{grad, (long)stride}, loss_sum, 0u, (float *)nullptr, scale_of(W, H), mg, g.tiles_x,
                       g.nb);
    return launched();
}

int sad_render_bwd_rec(const float *rec, int n_slots, const uint32_t *cand, const float *target, int W, int H,
                       int cell, float *grad, float *loss_sum, float *out_rgb, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || cell < 1)
        return SAD_ERR_ARG;
    if (W == 0 || H == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!rec && n_slots > 0) || !cand || !target || (!grad && n_slots > 0))
        return SAD_ERR_ARG;
    if (!aligned16(cand) || !aligned16(grad) || !aligned16(rec))
        return SAD_ERR_ALIGN;
    const TileGrid g = tile_grid(W, H);
    hipLaunchKernelGGL((k_render_bwd<SEL_REC, GL_REC>), dim3(g.nb), dim3(PAIR_THREADS), 0, (hipStream_t)stream,
                       src_of(rec), (uint32_t)n_slots, (const uint4 *)cand, target, W, H, GradOut{grad, 0}, loss_sum,
                       (uint32_t)(SAD_LOSS_SLOTS - 1), out_rgb, scale_of(W, H), mg, g.tiles_x, g.nb);
    return launched();
}

int sad_densify_stats(const float *rec, int n_slots, const uint32_t *cand, const float *target, int W, int H,
                      int cell, float *stats, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || cell < 1)
        return SAD_ERR_ARG;
    if (W == 0 || H == 0)
        return SAD_OK;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if ((!rec && n_slots > 0) || !cand || !target || (!stats && n_slots > 0))
        return SAD_ERR_ARG;
    if (!aligned16(cand) || !aligned16(rec) || !aligned16(stats))
        return SAD_ERR_ALIGN;
    const TileGrid g = tile_grid(W, H);
    hipLaunchKernelGGL(k_densify_stats, dim3(g.nb), dim3(BLOCK), 0, (hipStream_t)stream, src_of(rec),
                       (uint32_t)n_slots, (const uint4 *)cand, target, W, H, stats, scale_of(W, H), mg, g.tiles_x,
                       g.nb);
    return launched();
}

int sad_adam_step(float *sites, float *m, float *v, float *grad, int n_slots, int stride, int step, int n_pixels,
                  const sad_adam_cfg *cfg, void *stream)
{
    return adam_any(sites, m, v, grad, GL_PLANES, nullptr, nullptr, nullptr, n_slots, stride, step, n_pixels, cfg,
                    stream);
}

int sad_adam_step_rec(float *sites, float *m, float *v, float *grad, float *rec, uint32_t *packed, uint32_t *scr,
                      int n_slots, int stride, int step, int n_pixels, const sad_adam_cfg *cfg, void *stream)
{
    return adam_any(sites, m, v, grad, GL_REC, rec, packed, scr, n_slots, stride, step, n_pixels, cfg, stream);
}

int sad_eval_encode(const float *sites, int n_slots, int stride, int W, int H, uint32_t *words, float *header,
                    void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)) || (rc = check_image(W, H)))
        return rc;
    if (W < 1 || H < 1 || !header || (n_slots > 0 && (!sites || !words)))
        return SAD_ERR_ARG;
    if (!aligned16(words) || !aligned16(header))
        return SAD_ERR_ALIGN;
    const hipStream_t hs = (hipStream_t)stream;
    uint32_t *keys = reinterpret_cast<uint32_t *>(header);
    hipLaunchKernelGGL(k_eval_range_init, dim3(1), dim3(64), 0, hs, keys);
    if (n_slots > 0) {
        hipLaunchKernelGGL(k_eval_range, dim3((n_slots + 255) / 256), dim3(256), 0, hs, sites, n_slots, stride, keys);
        hipLaunchKernelGGL(k_eval_encode, dim3((n_slots + 255) / 256), dim3(256), 0, hs, sites, n_slots, stride,
                           (float)EV_QPOS / (float)W, (float)EV_QPOS / (float)H, (const uint32_t *)keys,
                           (uint4 *)words);
    }
    hipLaunchKernelGGL(k_eval_header, dim3(1), dim3(64), 0, hs, keys);
    return launched();
}

int sad_eval_decode(const uint32_t *words, const float *header, int n_slots, int W, int H, float *sites, int stride,
                    void *stream)
{
    int rc;
    if ((rc = check_sites(n_slots, stride)) || (rc = check_image(W, H)))
        return rc;
    if (W < 1 || H < 1)
        return SAD_ERR_ARG;
    if (n_slots == 0)
        return SAD_OK;
    if (!words || !header || !sites)
        return SAD_ERR_ARG;
    if (!aligned16(words) || !aligned16(header))
        return SAD_ERR_ALIGN;
    hipLaunchKernelGGL(k_eval_decode, dim3((n_slots + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)words, (const float4 *)header, n_slots, (float)W / (float)EV_QPOS,
                       (float)H / (float)EV_QPOS, sites, stride);
    return launched();
}

int sad_eval_query(const uint32_t *words, const float *header, int n_slots, const uint32_t *cand, int W, int H,
                   int cell, const float *points, int64_t n_points, float *out_rgb, void *stream)
{
    int rc;
    if ((rc = check_image(W, H)))
        return rc;
    if (n_slots < 0 || cell < 1 || n_points < 0 || W < 1 || H < 1)
        return SAD_ERR_ARG;
    MapGrid mg;
    int Wm, Hm;
    if (!map_grid(W, H, cell, mg, Wm, Hm))
        return SAD_ERR_ARG;
    if (n_points == 0)
        return SAD_OK;
    if (!header || !cand || !points || !out_rgb || (n_slots > 0 && !words))
        return SAD_ERR_ARG;
    if (!aligned16(words) || !aligned16(header) || !aligned16(cand) || ((uintptr_t)points & 7u))
        return SAD_ERR_ALIGN;
    if (n_points > (int64_t)0x7FFFFF00)  // one point per lane, at most 2^23 workgroups
        return SAD_ERR_ARG;
    hipLaunchKernelGGL(k_eval_query, dim3((unsigned)((n_points + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)words, (const float4 *)header, (uint32_t)n_slots, (const uint4 *)cand, W, H, mg,
                       (const float2 *)points, (long)n_points, out_rgb, scale_of(W, H), (float)W / (float)EV_QPOS,
                       (float)H / (float)EV_QPOS);
    return launched();
}

}  // extern "C"
