// Stages (a, gather) and (b): sorted box gather, then the triangle-tiled IoU
// suppression bitmask.
//
// Bitmask layout ("LeetCUDA 14-nms", Phase 1, with 64-bit words): row p of
// the mask belongs to sorted box p; bit l of its word for column tile c is 1
// iff box q = 64c + l comes after p (q > p), exists (q < n), is in p's group,
// and IoU(p, q) > t.  Bit l of word c means box 64c + l in every row, so the
// sweep can OR rows together; boxes at or before the row never vote (the
// page's j_base alignment with the lanes for j <= i voting 0).
//
// Mapping to gfx950.  One wave64 owns a work item: one row tile r (64 sorted
// boxes) against a strip of S consecutive column tiles.  Lane l holds column
// box 64c + l of each of the S tiles in VGPRs; the 64 row boxes are uniform,
// so they are read with scalar loads and broadcast from SGPRs.  For every
// row k the lanes evaluate their IoU test and the wave-wide compare mask is
// the 64-bit mask word itself (a ballot, as the page's warp vote, but 64
// wide).  Lane k keeps row k's words, and after the strip each lane stores
// its S words (S * 8 bytes, one full 128-byte line for S = 16) contiguously.
// Tiles left of the diagonal are skipped (the triangle skip of the Matrix NMS
// page's tiling and of the tile kernel of "nms_kernel.cu analysis 2") and
// written as zeros; in the diagonal tile only lanes l > k vote.  There is no
// matrix-core (MFMA) use: nothing here is a dense contraction.
//
// Threshold test.  The mask must agree bit for bit with the float32
// expression "inter / union > t".  When every box has a finite area > 0
// (checked by the gather kernel), 0 <= inter <= union and union > 0, and
// the test is exactly equivalent to comparing inter against m * union in
// binary64, where m = t + ulp(t)/2 is the rounding boundary above t: the
// product of a 25-bit m and a 24-bit union is exact in binary64, and the
// float32 quotient exceeds t iff the real quotient reaches m (ties at m round
// up when t's last significand bit is odd, to t when it is even).  That costs
// two conversions, one multiply and one compare instead of a correctly
// rounded division.  Otherwise (degenerate or inverted boxes, t <= 0) the
// kernel performs the literal float32 division.
#include <cmath>
#include <cstring>

#include "nms_internal.h"

#pragma clang fp contract(off)

namespace gnms {
namespace {

enum TestMode { MODE_EVEN = 0, MODE_ODD = 1, MODE_LITERAL = 2 };

template <int MODE>
__device__ __forceinline__ bool exceeds(float inter, float uni, float t, double mid) {
    if (MODE == MODE_LITERAL) {
        const float iou = inter / uni;
        return iou > t;
    } else {
        const double lhs = (double)inter;
        const double rhs = mid * (double)uni;
        return MODE == MODE_ODD ? lhs >= rhs : lhs > rhs;
    }
}

// max and min of finite floats as v_med3_f32 against +-infinity: med3(a, b,
// +inf) = max(a, b) and med3(a, b, -inf) = min(a, b) for non-NaN a, b.  The
// infinities arrive as kernel arguments, so the compiler cannot fold the
// median back into fmaxf/fminf, which in the IEEE mode kernels run in must
// first quiet possible signalling NaNs (an extra instruction per operand and
// use).  Coordinates are checked finite before a result is accepted, and the
// sign of a zero (the only thing these forms might treat differently) never
// changes a decision.
__device__ __forceinline__ float max2(float a, float b, float pinf) {
    return __builtin_amdgcn_fmed3f(a, b, pinf);
}
__device__ __forceinline__ float min2(float a, float b, float ninf) {
    return __builtin_amdgcn_fmed3f(a, b, ninf);
}

template <int MODE>
__device__ __forceinline__ bool suppresses(float rx1, float ry1, float rx2, float ry2, float ra,
                                           float cx1, float cy1, float cx2, float cy2, float ca,
                                           float t, double mid, float pinf, float ninf) {
    const float xx1 = max2(rx1, cx1, pinf);
    const float yy1 = max2(ry1, cy1, pinf);
    const float xx2 = min2(rx2, cx2, ninf);
    const float yy2 = min2(ry2, cy2, ninf);
    const float w = max2(xx2 - xx1, 0.0f, pinf);
    // The division-free tests (positive areas, t > 0) need only one clamp:
    // with w >= 0 and h unclamped, boxes that do not overlap give w * h <= 0
    // (a zero or negative product, never above m * union > 0), so the
    // decision is the same as with max(h, 0); boxes that overlap give the
    // very product of the definition.  The literal test keeps both clamps.
    const float dh = yy2 - yy1;
    const float h = MODE == MODE_LITERAL ? max2(dh, 0.0f, pinf) : dh;
    const float inter = w * h;
    const float uni = (ra + ca) - inter;
    return exceeds<MODE>(inter, uni, t, mid);
}

// ---------------------------------------------------------------- gather

struct GatherArgs {
    const float4 *boxes;
    int n, npad, words, grouped;
    Work w;
};

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= a.npad) return;
    if (p < a.words) a.w.tcount[p] = 0u;  // the mask kernel counts each tile's nonzero words
    // near words stay 0 where the tile lies outside the row's band
    for (int j = 0; j <= NEAR_TILES; ++j) a.w.tnear[(size_t)j * a.npad + p] = 0ull;
    bool finite = true, positive = true;
    if (p < a.n) {
        const int i = a.w.order[p];
        const float4 b = a.boxes[i];
        finite = isfinite(b.x) && isfinite(b.y) && isfinite(b.z) && isfinite(b.w);
        const float ar = (b.z - b.x) * (b.w - b.y);
        positive = ar > 0.0f && ar < INFINITY;
        a.w.sb[p] = b;
        a.w.area[p] = ar;
        if (a.grouped) a.w.inv[i] = p;
    } else {
        a.w.sb[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        a.w.area[p] = 0.0f;
    }
    const uint64_t bad_f = __ballot(!finite);
    const uint64_t bad_a = __ballot(!positive);
    if ((threadIdx.x & 63) == 0) {
        if (bad_f) atomicOr(&a.w.ctrl->error, ERR_NONFINITE);
        if (bad_a) atomicAnd(&a.w.ctrl->flags, ~FLAG_POSITIVE_AREAS);
    }
}

// ---------------------------------------------------------------- mask

struct MaskArgs {
    int n, words, mstride, npad;
    float t;
    double mid;
    int odd, exact_ok;
    float pinf, ninf;  // +inf and -inf, see max2/min2
};

// Read-only inputs and the output of the mask kernel.  They are separate
// __restrict__ kernel parameters so the compiler can prove the uniform row
// loads never alias the mask stores and serve them from the scalar cache.
struct MaskPtrs {
    const float4 *__restrict__ sb;
    const float *__restrict__ area;
    const uint32_t *__restrict__ seg;
    const int32_t *__restrict__ tile_cend;
    const int32_t *__restrict__ item_base;
    uint64_t *__restrict__ mask;
    uint32_t *__restrict__ tcount;
    uint32_t *__restrict__ tent_wk;
    uint64_t *__restrict__ tent_val;
    uint64_t *__restrict__ tnear;
};

// v_writelane_b32: lane `lane` of the returned VGPR value becomes `val` (an
// SGPR); every other lane keeps `old`.  Used to park row k's mask word in
// lane k without touching the execution mask.
__device__ __forceinline__ uint32_t write_lane(uint32_t old, uint32_t val, int lane) {
    asm("v_writelane_b32 %0, %1, m0" : "+v"(old) : "s"(val), "{m0}"(lane));
    return old;
}

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// Word mask of valid column boxes in tile c (boxes >= n never vote).
__device__ __forceinline__ uint64_t column_valid(int c, int n) {
    const int rem = n - 64 * c;
    return rem >= 64 ? ~0ull : ((1ull << rem) - 1ull);
}

template <int S, bool GROUPED, int MODE>
__device__ __forceinline__ void mask_item(const MaskArgs &a, const MaskPtrs &m_, int item,
                                          int stride) {
    const int lane = threadIdx.x & 63;
    // row tile of this item: the largest r with item_base[r] <= item
    int lo = 0, hi = a.words - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (m_.item_base[mid] <= item) lo = mid;
        else hi = mid - 1;
    }
    const int r = lo;
    const int s0 = r / S;
    const int c0 = (s0 + (item - m_.item_base[r])) * S;
    const int cend = m_.tile_cend[r];
    const int p0 = 64 * r;
    const int rows = a.n - p0 < 64 ? a.n - p0 : 64;
    const int t_diag = r - c0;  // the diagonal tile's slot, if it lies in this strip

    // Column boxes of the strip, one per lane and tile.  Tiles outside
    // [r, cend) are evaluated on real boxes and masked out (tmask = 0), which
    // costs less than branching around them.
    float cx1[S], cy1[S], cx2[S], cy2[S], ca[S];
    uint32_t cg[S];
    uint64_t tmask[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
        const int c = c0 + t;
        const bool active = c >= r && c < cend;
        const int q = active ? 64 * c + lane : lane;
        const float4 b = m_.sb[q];
        cx1[t] = b.x;
        cy1[t] = b.y;
        cx2[t] = b.z;
        cy2[t] = b.w;
        ca[t] = m_.area[q];
        if (GROUPED) cg[t] = m_.seg[q];
        tmask[t] = active ? column_valid(c, a.n) : 0ull;
    }
    uint32_t out_lo[S], out_hi[S];
#pragma unroll
    for (int t = 0; t < S; ++t) out_lo[t] = out_hi[t] = 0u;

    for (int k = 0; k < rows; ++k) {
        const int p = p0 + k;
        const float4 rb = m_.sb[p];
        const float rx1 = rb.x;
        const float ry1 = rb.y;
        const float rx2 = rb.z;
        const float ry2 = rb.w;
        const float ra = m_.area[p];
        const uint32_t rg = GROUPED ? m_.seg[p] : 0u;
        // in the diagonal tile only boxes after row k vote
        const uint64_t dmask = k == 63 ? 0ull : (~0ull << (k + 1));
#pragma unroll
        for (int t = 0; t < S; ++t) {
            bool pred = suppresses<MODE>(rx1, ry1, rx2, ry2, ra, cx1[t], cy1[t], cx2[t], cy2[t],
                                         ca[t], a.t, a.mid, a.pinf, a.ninf);
            if (GROUPED) pred = pred && (cg[t] == rg);
            uint64_t m = __ballot(pred) & tmask[t];
            m &= (t == t_diag) ? dmask : ~0ull;
            out_lo[t] = write_lane(out_lo[t], (uint32_t)m, k);
            out_hi[t] = write_lane(out_hi[t], (uint32_t)(m >> 32), k);
        }
    }
    if (lane < rows) {
        const int p = p0 + lane;
        uint64_t *dst = m_.mask + (size_t)p * (size_t)stride + (size_t)(c0 - s0 * S);
        uint4 *d4 = reinterpret_cast<uint4 *>(dst);
#pragma unroll
        for (int t = 0; t < S; t += 2)
            d4[t / 2] = make_uint4(out_lo[t], out_hi[t], out_lo[t + 1], out_hi[t + 1]);
        // transposed copies of the words for tiles r .. r + NEAR_TILES
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const int j = t - t_diag;
            if (j >= 0 && j <= NEAR_TILES && c0 + t < cend)
                m_.tnear[(size_t)j * a.npad + p] = ((uint64_t)out_hi[t] << 32) | out_lo[t];
        }
    }
    // Record the strip's nonzero words in the row tile's list.  A wave-wide
    // prefix sum gives each lane its place and one atomic claims the wave's
    // slots, so the list order may differ from run to run; the sweep only ORs
    // entries together, which does not depend on their order.  Entries past
    // the capacity are dropped and the count (which still grows) tells the
    // sweep to read dense rows instead.
    uint32_t nz = 0;
    if (lane < rows) {
#pragma unroll
        for (int t = 0; t < S; ++t) nz += (out_lo[t] | out_hi[t]) != 0u;
    }
    const uint32_t incl = wave_incl_sum(nz);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    if (total) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&m_.tcount[r], total);
        base = __builtin_amdgcn_readlane(base, 0);
        uint32_t at = base + incl - nz;
#pragma unroll
        for (int t = 0; t < S; ++t) {
            if ((out_lo[t] | out_hi[t]) != 0u && lane < rows) {
                if (at < (uint32_t)TILE_LIST_CAP) {
                    const size_t e = (size_t)r * TILE_LIST_CAP + at;
                    m_.tent_wk[e] = ((uint32_t)(c0 + t) << 6) | (uint32_t)lane;
                    m_.tent_val[e] = ((uint64_t)out_hi[t] << 32) | out_lo[t];
                }
                ++at;
            }
        }
    }
}

template <int S, bool GROUPED>
__global__ __launch_bounds__(MASK_THREADS) void mask_kernel(
    MaskArgs a, const Ctrl *__restrict__ ctrl, const float4 *__restrict__ sb,
    const float *__restrict__ area, const uint32_t *__restrict__ seg,
    const int32_t *__restrict__ tile_cend, const int32_t *__restrict__ item_base,
    uint64_t *__restrict__ mask, uint32_t *__restrict__ tcount, uint32_t *__restrict__ tent_wk,
    uint64_t *__restrict__ tent_val, uint64_t *__restrict__ tnear) {
    const MaskPtrs m_{sb, area, seg, tile_cend, item_base, mask, tcount, tent_wk, tent_val, tnear};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves_per_block = MASK_THREADS / 64;
    const int num_items = ctrl->num_items;
    const bool fast = (ctrl->flags & FLAG_POSITIVE_AREAS) && a.exact_ok;
    const int stride = GROUPED ? ctrl->band_stride : a.mstride;
    for (int item = blockIdx.x * waves_per_block + wave; item < num_items;
         item += gridDim.x * waves_per_block) {
        if (fast) {
            if (a.odd) mask_item<S, GROUPED, MODE_ODD>(a, m_, item, stride);
            else mask_item<S, GROUPED, MODE_EVEN>(a, m_, item, stride);
        } else {
            mask_item<S, GROUPED, MODE_LITERAL>(a, m_, item, stride);
        }
    }
}

// ---------------------------------------------------------------- decide

__global__ void decide_kernel(const float *inter, const float *uni, int64_t count, float t,
                              double mid, int mode, uint8_t *out) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= count) return;
    bool r;
    if (mode == MODE_EVEN) r = exceeds<MODE_EVEN>(inter[k], uni[k], t, mid);
    else if (mode == MODE_ODD) r = exceeds<MODE_ODD>(inter[k], uni[k], t, mid);
    else r = exceeds<MODE_LITERAL>(inter[k], uni[k], t, mid);
    out[k] = r ? 1 : 0;
}

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

}  // namespace

Threshold make_threshold(float t) {
    Threshold th;
    th.t = t;
    th.exact_ok = std::isfinite(t) && t > 0.0f;
    th.mid = 0.0;
    th.odd = false;
    if (th.exact_ok) {
        uint32_t bits;
        memcpy(&bits, &t, sizeof(bits));
        th.odd = (bits & 1u) != 0;
        int e = 0;
        std::frexp(t, &e);  // t = f * 2^e, f in [0.5, 1)
        double ulp = std::ldexp(1.0, e - 24);
        const double min_ulp = std::ldexp(1.0, -149);
        if (ulp < min_ulp) ulp = min_ulp;
        th.mid = (double)t + ulp / 2.0;
    }
    return th;
}

hipError_t launch_gather(const Problem &P, const Layout &L, const Work &w, hipStream_t stream) {
    GatherArgs a;
    a.boxes = reinterpret_cast<const float4 *>(P.boxes);
    a.n = P.n;
    a.npad = (int)L.npad;
    a.words = (int)L.words;
    a.grouped = P.grouped ? 1 : 0;
    a.w = w;
    const int blocks = (int)((L.npad + 255) / 256);
    hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_mask(const Problem &P, const Layout &L, const Work &w, hipStream_t stream) {
    const Threshold th = make_threshold(P.thresh);
    MaskArgs a;
    a.n = P.n;
    a.npad = (int)L.npad;
    a.words = (int)L.words;
    a.mstride = (int)L.mstride;
    a.t = th.t;
    a.mid = th.mid;
    a.odd = th.odd ? 1 : 0;
    a.exact_ok = th.exact_ok ? 1 : 0;
    a.pinf = INFINITY;
    a.ninf = -INFINITY;
    // Upper bound on work items: every row tile covers all strips to the end.
    const int64_t W = L.words;
    const int S = P.strip;
    int64_t items_ub = 0;
    for (int64_t r = 0; r < W; r += S) {
        const int64_t rows_here = (r + S <= W) ? S : (W - r);
        items_ub += rows_here * ((W + S - 1) / S - r / S);
    }
    const int waves_per_block = MASK_THREADS / 64;
    int64_t blocks = (items_ub + waves_per_block - 1) / waves_per_block;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    if (P.grouped)
        hipLaunchKernelGGL((mask_kernel<STRIP_GROUPED, true>), dim3((unsigned)blocks),
                           dim3(MASK_THREADS), 0, stream, a, w.ctrl, w.sb, w.area, w.seg,
                           w.tile_cend, w.item_base, w.mask, w.tcount, w.tent_wk, w.tent_val,
                           w.tnear);
    else
        hipLaunchKernelGGL((mask_kernel<STRIP_SINGLE, false>), dim3((unsigned)blocks),
                           dim3(MASK_THREADS), 0, stream, a, w.ctrl, w.sb, w.area, w.seg,
                           w.tile_cend, w.item_base, w.mask, w.tcount, w.tent_wk, w.tent_val,
                           w.tnear);
    return hipGetLastError();
}

hipError_t launch_decide(const float *inter, const float *uni, int64_t count, float thresh,
                         bool positive_areas, uint8_t *out, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const Threshold th = make_threshold(thresh);
    int mode = MODE_LITERAL;
    if (positive_areas && th.exact_ok) mode = th.odd ? MODE_ODD : MODE_EVEN;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(decide_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, inter, uni,
                       count, thresh, th.mid, mode, out);
    return hipGetLastError();
}

}  // namespace gnms
