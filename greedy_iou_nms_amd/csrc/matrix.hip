// Matrix NMS with the Gaussian decay ("Fastest Matrix NMS in the West (Part
// 2)": "What do we need to compute?" and optimisations 1, 2 and 4), on the
// sorted boxes the radix sort leaves in the workspace.
//
// With the boxes in descending score order, O[p][q] (p < q) is the IoU of
// father p and child q, omax[q] the largest O[p][q] over q's fathers, and a
// child is dropped when its score is below the threshold t or some father
// gives a candidate decayed score below it:
//     exp((omax[p]^2 - O[p][q]^2) / sigma) * s_q  <  t.
// The IoUs are the library's float32 expression (0/0 counted as 0); the decay
// test is decided in binary64.
//
//   matrix_prep_kernel          per sorted position: its score, the box-order
//                               check, the inverse order for the compaction,
//                               and the fast-path bounds of its decay test.
//   matrix_overlap_max_kernel   triangle-tiled like the suppression mask: one
//                               wave per (row tile of fathers, strip of MS
//                               child tiles); lane l holds child 64c + l of
//                               each tile, father rows come from scalar loads;
//                               each lane keeps its running maximum and
//                               raises omax[q] with one atomic max per tile
//                               (the page's fused first reduction; later
//                               passes are not needed with atomics).
//   matrix_decay_kernel         the same tiling; per pair the IoU again (the
//                               page stores the N x N matrix; recomputing it
//                               costs less than writing and reading it back)
//                               and D = omax[p]^2 - O^2 in binary64.  The test
//                               "exp(D / sigma) s_q < t" is, for s_q > 0 and
//                               t > 0, "D < sigma ln(t / s_q)"; a pair with D
//                               clear of that bound by 1e-9 (sigma + 1) is
//                               decided at once, a pair inside that margin by
//                               evaluating the literal expression (rare), so
//                               the decision is the literal one.  Dropped
//                               children are ORed into a bitmap per tile (the
//                               page's drop flags, one atomic per tile).
//   matrix_keep_kernel          kept bitmap = score at least t and not dropped.
#include <cmath>

#include "nms_internal.h"

#pragma clang fp contract(off)

namespace gnms {
namespace {

constexpr int MS = 8;        // child tiles per work item
constexpr int MT = 256;      // threads per workgroup
constexpr int MWAVES = MT / 64;

struct MatrixArgs {
    const float4 *__restrict__ sb;
    const float *__restrict__ area;
    const float *__restrict__ mscore;
    uint32_t *momax;
    const double *__restrict__ mlo;
    const double *__restrict__ mhi;
    uint64_t *mdrop;
    const Ctrl *ctrl;
    int n, words, qshift;
    float t;
    double sigma;
};

// First work item of row tile r when every row covers all child tiles up to
// W: strips floor(r/S) .. ceil(W/S)-1.
__host__ __device__ __forceinline__ int item_base(int r, int W) {
    const int G = (W + MS - 1) / MS;
    const int g = r / MS, u = r % MS;
    return MS * (g * G - g * (g - 1) / 2) + u * (G - g);
}

struct Item {
    int r, c0, k_lo, k_hi;
};

__device__ __forceinline__ Item decode(const MatrixArgs &a, int item) {
    const int rpi = 64 >> a.qshift;
    const int pair = item >> a.qshift;
    int lo = 0, hi = a.words - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (item_base(mid, a.words) <= pair) lo = mid;
        else hi = mid - 1;
    }
    Item it;
    it.r = lo;
    it.c0 = (lo / MS + (pair - item_base(lo, a.words))) * MS;
    it.k_lo = (item & ((1 << a.qshift) - 1)) * rpi;
    const int tile_rows = a.n - 64 * lo < 64 ? a.n - 64 * lo : 64;
    it.k_hi = it.k_lo + rpi < tile_rows ? it.k_lo + rpi : tile_rows;
    return it;
}

// The library's float32 IoU of a father (r) and a child (c), 0/0 counted as
// 0.  Boxes are ordered (x1 <= x2, y1 <= y2, checked by the prep kernel), so
// clamping the child's coordinates into the father's extent gives the
// definition's max/min intersection bit for bit (zero where they do not
// overlap); the quotient is the correctly rounded division, and fmaxf turns
// the only possible NaN (0/0: both boxes empty) into 0.
__device__ __forceinline__ float overlap(float rx1, float ry1, float rx2, float ry2, float ra,
                                         float cx1, float cy1, float cx2, float cy2, float ca) {
    const float xx1 = __builtin_amdgcn_fmed3f(cx1, rx1, rx2);
    const float xx2 = __builtin_amdgcn_fmed3f(cx2, rx1, rx2);
    const float yy1 = __builtin_amdgcn_fmed3f(cy1, ry1, ry2);
    const float yy2 = __builtin_amdgcn_fmed3f(cy2, ry1, ry2);
    const float inter = (xx2 - xx1) * (yy2 - yy1);
    const float uni = (ra + ca) - inter;
    return fmaxf(inter / uni, 0.0f);
}

// Sign words of the four edge differences, ORed: a clear sign bit is
// necessary for a positive intersection (boxes are ordered, and a float
// difference keeps the sign of the exact one, a tie giving +0), so a pair
// whose word has its sign bit set has O = 0.
__device__ __forceinline__ uint32_t may_overlap(float rx1, float ry1, float rx2, float ry2,
                                                float cx1, float cy1, float cx2, float cy2) {
    return __float_as_uint(rx2 - cx1) | __float_as_uint(cx2 - rx1) |
           __float_as_uint(ry2 - cy1) | __float_as_uint(cy2 - ry1);
}

// child tiles per may-overlap question (measured at 65,536 boxes: the
// maximum takes 0.30-0.33 ms asking per 2 tiles, 0.37-0.39 per 4 and
// 0.31-0.32 per tile, where the decay step is slower)
constexpr int MG = 2;

struct Children {
    float x1[MS], y1[MS], x2[MS], y2[MS], a[MS];
    uint64_t valid[MS];  // lanes that are real children of this item's tile
};

__device__ __forceinline__ void load_children(const MatrixArgs &a, const Item &it, Children &ch) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < MS; ++t) {
        const int c = it.c0 + t;
        const bool active = c >= it.r && c < a.words;
        const int q = active ? 64 * c + lane : lane;
        const float4 b = a.sb[q];
        ch.x1[t] = b.x;
        ch.y1[t] = b.y;
        ch.x2[t] = b.z;
        ch.y2[t] = b.w;
        ch.a[t] = a.area[q];
        const int left = a.n - 64 * c;
        ch.valid[t] = !active ? 0ull : left >= 64 ? ~0ull : (left <= 0 ? 0ull : (1ull << left) - 1ull);
    }
}

// Running maxima of one item's rows.  A pair with no overlap has O = 0 and
// leaves a maximum (which starts at 0) as it is, so each group of MG child
// tiles first asks whether any lane may overlap in any of them, and only the
// tiles where some lane may overlap compute their IoUs.  In the diagonal
// item (DIAG) only children after the father count in the diagonal tile;
// elsewhere every child tile lies after the father's tile, and lanes that
// are no child hold an empty box (O = 0).
template <bool DIAG>
__device__ __forceinline__ void max_rows(const MatrixArgs &a, const Item &it, const Children &ch,
                                         float (&m)[MS]) {
    const int lane = threadIdx.x & 63;
    const int t_diag = it.r - it.c0;
    for (int k = it.k_lo; k < it.k_hi; ++k) {
        const int p = 64 * it.r + k;
        const float4 rb = a.sb[p];
        const float ra = a.area[p];
        const bool after = lane > k;
#pragma unroll
        for (int t0 = 0; t0 < MS; t0 += MG) {
            uint32_t sgn[MG];
            uint32_t all = ~0u;
#pragma unroll
            for (int j = 0; j < MG; ++j) {
                const int t = t0 + j;
                sgn[j] = may_overlap(rb.x, rb.y, rb.z, rb.w, ch.x1[t], ch.y1[t], ch.x2[t],
                                     ch.y2[t]);
                all &= sgn[j];
            }
            if (__ballot((int32_t)all >= 0) == 0ull) continue;
#pragma unroll
            for (int j = 0; j < MG; ++j) {
                const int t = t0 + j;
                if (__ballot((int32_t)sgn[j] >= 0) == 0ull) continue;
                const float o = overlap(rb.x, rb.y, rb.z, rb.w, ra, ch.x1[t], ch.y1[t],
                                        ch.x2[t], ch.y2[t], ch.a[t]);
                const float mo = fmaxf(m[t], o);
                m[t] = (!DIAG || t != t_diag || after) ? mo : m[t];
            }
        }
    }
}

__global__ __launch_bounds__(MT) void matrix_overlap_max_kernel(MatrixArgs a, int num_items) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int slots = gridDim.x * MWAVES;
    for (int item = blockIdx.x * MWAVES + wave; item < num_items; item += slots) {
        const Item it = decode(a, item);
        Children ch;
        load_children(a, it, ch);
        const int t_diag = it.r - it.c0;
        float m[MS];
#pragma unroll
        for (int t = 0; t < MS; ++t) m[t] = 0.0f;
        if (t_diag >= 0 && t_diag < MS) max_rows<true>(a, it, ch, m);
        else max_rows<false>(a, it, ch, m);
#pragma unroll
        for (int t = 0; t < MS; ++t) {
            // omax holds non-negative floats, whose bit patterns order as
            // unsigned integers
            if (((ch.valid[t] >> lane) & 1ull) && m[t] > 0.0f)
                atomicMax(&a.momax[64 * (it.c0 + t) + lane], __float_as_uint(m[t]));
        }
    }
}

// The literal test of a pair inside the margin, out of line: inlined, the
// binary64 exp's registers raised the decay kernel to 155 VGPRs (3 waves per
// SIMD); with the call (rarely taken) and a 4-wave hint it fits 128.
__device__ __attribute__((noinline)) bool literal_drop(double x, double s, double t) {
    return exp(x) * s < t;
}

// The decay test of one pair for the MS child tiles of tile t: D = omax[p]^2
// - O^2 against the child's bounds, the literal expression inside the
// margin; returns the lanes that drop.
__device__ __forceinline__ uint64_t decay_drops(const MatrixArgs &a, const Item &it,
                                                const Children &ch, int t, float4 rb, float ra,
                                                double A, double lo, double hi, uint64_t live,
                                                double t64) {
    const int lane = threadIdx.x & 63;
    const float o = overlap(rb.x, rb.y, rb.z, rb.w, ra, ch.x1[t], ch.y1[t], ch.x2[t], ch.y2[t],
                            ch.a[t]);
    const double od = (double)o;
    const double D = __builtin_fma(-od, od, A);
    uint64_t sure = __ballot(D < lo);
    const uint64_t unsure = __ballot(D < hi) & ~sure;
    if (unsure & live) {
        // within the margin: the literal expression
        const int q = 64 * (it.c0 + t) + lane;
        bool hit = false;
        if ((unsure >> lane) & 1ull) {
            const double x = (A - od * od) / a.sigma;
            hit = literal_drop(x, (double)a.mscore[q], t64);
        }
        sure |= __ballot(hit);
    }
    return sure & live;
}

// The rows of one item.  SKIP: no child of this call has a negative score at
// or above t, so a pair with no overlap never drops its child: it has D =
// omax[p]^2 >= 0 and exp(D / sigma) s_q >= s_q >= t for s_q >= 0, and
// children below t are dropped by the keep step anyway.  Groups of MG child
// tiles where no lane may overlap are then skipped, as in the maximum.
template <bool SKIP>
__device__ __forceinline__ void decay_rows(const MatrixArgs &a, const Item &it,
                                           const Children &ch, const double (&lo)[MS],
                                           const double (&hi)[MS], uint64_t (&drop)[MS]) {
    const double t64 = (double)a.t;
    const int t_diag = it.r - it.c0;
    for (int k = it.k_lo; k < it.k_hi; ++k) {
        const int p = 64 * it.r + k;
        const float4 rb = a.sb[p];
        const float ra = a.area[p];
        const float om = __uint_as_float(a.momax[p]);
        const double A = (double)om * (double)om;  // exact: 24 x 24 bits
        const uint64_t after = k == 63 ? 0ull : (~0ull << (k + 1));
#pragma unroll
        for (int t0 = 0; t0 < MS; t0 += MG) {
            uint32_t sgn[MG];
            if (SKIP) {
                uint32_t all = ~0u;
#pragma unroll
                for (int j = 0; j < MG; ++j) {
                    const int t = t0 + j;
                    sgn[j] = may_overlap(rb.x, rb.y, rb.z, rb.w, ch.x1[t], ch.y1[t], ch.x2[t],
                                         ch.y2[t]);
                    all &= sgn[j];
                }
                if (__ballot((int32_t)all >= 0) == 0ull) continue;
            }
#pragma unroll
            for (int j = 0; j < MG; ++j) {
                const int t = t0 + j;
                if (SKIP && __ballot((int32_t)sgn[j] >= 0) == 0ull) continue;
                const uint64_t live = ch.valid[t] & (t == t_diag ? after : ~0ull);
                drop[t] |= decay_drops(a, it, ch, t, rb, ra, A, lo[t], hi[t], live, t64);
            }
        }
    }
}

__global__ __launch_bounds__(MT) __attribute__((amdgpu_waves_per_eu(4))) void matrix_decay_kernel(
    MatrixArgs a, int num_items) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int slots = gridDim.x * MWAVES;
    const bool skip = !(a.ctrl->flags & FLAG_MATRIX_ZERO_PAIRS_MATTER);
    for (int item = blockIdx.x * MWAVES + wave; item < num_items; item += slots) {
        const Item it = decode(a, item);
        Children ch;
        load_children(a, it, ch);
        double lo[MS], hi[MS];
#pragma unroll
        for (int t = 0; t < MS; ++t) {
            const int c = it.c0 + t;
            const int q = (c >= it.r && c < a.words) ? 64 * c + lane : lane;
            lo[t] = a.mlo[q];
            hi[t] = a.mhi[q];
        }
        uint64_t drop[MS];
#pragma unroll
        for (int t = 0; t < MS; ++t) drop[t] = 0ull;
        if (skip) decay_rows<true>(a, it, ch, lo, hi, drop);
        else decay_rows<false>(a, it, ch, lo, hi, drop);
#pragma unroll
        for (int t = 0; t < MS; ++t)
            if (drop[t] && lane == 0) atomicOr(&a.mdrop[it.c0 + t], drop[t]);
    }
}

struct PrepArgs {
    const float *scores;
    const int32_t *order;
    const float4 *sb;
    float *mscore;
    uint32_t *momax;
    double *mlo, *mhi;
    uint64_t *mdrop;
    int32_t *inv;
    int32_t *score_order;
    Ctrl *ctrl;
    int n, npad, words;
    float t;
    double sigma;
};

__global__ __launch_bounds__(256) void matrix_prep_kernel(PrepArgs a) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p < a.words) a.mdrop[p] = 0ull;
    if (p >= a.npad) return;
    double lo = -INFINITY, hi = -INFINITY;
    float s = 0.0f;
    bool bad = false, neg = false;
    if (p < a.n) {
        const int32_t i = a.order[p];
        s = a.scores[i];
        a.inv[i] = p;
        a.score_order[p] = i;
        const float4 b = a.sb[p];
        bad = b.x > b.z || b.y > b.w;
        const double sd = (double)s, td = (double)a.t;
        if (!(sd < td)) {  // a score below t drops the box whatever its fathers
            if (sd > 0.0 && td > 0.0) {
                const double bound = a.sigma * log(td / sd);
                const double margin = 1e-9 * (a.sigma + 1.0);
                lo = bound - margin;
                hi = bound + margin;
            } else if (sd < 0.0) {
                // t <= s < 0: every pair by the literal expression, and a
                // father with no overlap can drop the child
                hi = INFINITY;
                neg = true;
            }
            // s >= 0 >= t (s = 0 or t <= 0 < s): no candidate falls below t
        }
    }
    a.mscore[p] = s;
    a.momax[p] = 0u;
    a.mlo[p] = lo;
    a.mhi[p] = hi;
    const uint64_t any_bad = __ballot(bad);
    if (any_bad && (threadIdx.x & 63) == 0) atomicOr(&a.ctrl->error, ERR_BAD_BOXES);
    const uint64_t any_neg = __ballot(neg);
    if (any_neg && (threadIdx.x & 63) == 0)
        atomicOr(&a.ctrl->flags, FLAG_MATRIX_ZERO_PAIRS_MATTER);
}

__global__ __launch_bounds__(256) void matrix_keep_kernel(const float *mscore,
                                                          const uint64_t *mdrop, uint64_t *kept,
                                                          int n, int words, float t) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    const int w = p >> 6;
    const bool keep = p < n && !(mscore[p] < t) && !((mdrop[w < words ? w : 0] >> (p & 63)) & 1ull);
    const uint64_t m = __ballot(keep);
    if ((threadIdx.x & 63) == 0 && w < words) kept[w] = m;
}

MatrixArgs make_args(const Problem &P, const Layout &L, const Work &w, double sigma) {
    MatrixArgs a;
    a.sb = w.sb;
    a.area = w.area;
    a.mscore = w.mscore;
    a.momax = w.momax;
    a.mlo = w.mlo;
    a.mhi = w.mhi;
    a.mdrop = w.mdrop;
    a.ctrl = w.ctrl;
    a.n = P.n;
    a.words = (int)L.words;
    a.t = P.thresh;
    a.sigma = sigma;
    // split each (row tile, strip) pair into up to 4 items when there are
    // too few pairs to give every resident wave one
    const int64_t pairs = (int64_t)item_base((int)L.words, (int)L.words);
    const int64_t slots = (int64_t)device_cu_count() * 16;
    a.qshift = 0;
    while (a.qshift < 2 && (pairs << a.qshift) < slots) ++a.qshift;
    return a;
}

hipError_t launch_items(void (*kernel)(MatrixArgs, int), const MatrixArgs &a, int64_t pairs,
                        hipStream_t stream) {
    const int64_t items = pairs << a.qshift;
    int64_t blocks = (items + MWAVES - 1) / MWAVES;
    if (blocks > MAX_GRID_THREADS / MT) blocks = MAX_GRID_THREADS / MT;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(MT), 0, stream, a, (int)items);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_matrix_prep(const Problem &P, const Layout &L, const Work &w, double sigma,
                              hipStream_t stream) {
    PrepArgs a;
    a.scores = P.scores;
    a.order = w.order;
    a.sb = w.sb;
    a.mscore = w.mscore;
    a.momax = w.momax;
    a.mlo = w.mlo;
    a.mhi = w.mhi;
    a.mdrop = w.mdrop;
    a.inv = w.inv;
    a.score_order = w.score_order;
    a.ctrl = w.ctrl;
    a.n = P.n;
    a.npad = (int)L.npad;
    a.words = (int)L.words;
    a.t = P.thresh;
    a.sigma = sigma;
    hipLaunchKernelGGL(matrix_prep_kernel, dim3((unsigned)((L.npad + 255) / 256)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_matrix_overlap_max(const Problem &P, const Layout &L, const Work &w,
                                     hipStream_t stream) {
    const MatrixArgs a = make_args(P, L, w, 1.0);
    return launch_items(matrix_overlap_max_kernel, a, item_base((int)L.words, (int)L.words),
                        stream);
}

hipError_t launch_matrix_decay(const Problem &P, const Layout &L, const Work &w, double sigma,
                               hipStream_t stream) {
    const MatrixArgs a = make_args(P, L, w, sigma);
    hipError_t e =
        launch_items(matrix_decay_kernel, a, item_base((int)L.words, (int)L.words), stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(matrix_keep_kernel, dim3((unsigned)((L.npad + 255) / 256)), dim3(256), 0,
                       stream, w.mscore, w.mdrop, w.kept, P.n, (int)L.words, P.thresh);
    return hipGetLastError();
}

}  // namespace gnms
