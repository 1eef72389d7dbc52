// The per-item IoU mask computation, shared by the standalone mask kernel
// (mask.hip, which also describes the bitmask layout, the mapping to
// gfx950 and the division-free threshold test) and the fused mask + sweep
// kernel (sweep.hip).
#pragma once

#include <cmath>

#include "nms_internal.h"

#pragma clang fp contract(off)

namespace gnms {
namespace maskcore {

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

// Intersection area of ordered boxes (x1 < x2, y1 < y2), as described in
// suppresses() below: the column box clamped into the row box's extent.
__device__ __forceinline__ float intersection(float rx1, float ry1, float rx2, float ry2,
                                              float cx1, float cy1, float cx2, float cy2) {
    const float xx1 = __builtin_amdgcn_fmed3f(cx1, rx1, rx2);
    const float xx2 = __builtin_amdgcn_fmed3f(cx2, rx1, rx2);
    const float yy1 = __builtin_amdgcn_fmed3f(cy1, ry1, ry2);
    const float yy2 = __builtin_amdgcn_fmed3f(cy2, ry1, ry2);
    return (xx2 - xx1) * (yy2 - yy1);
}

template <int MODE>
__device__ __forceinline__ bool suppresses(float rx1, float ry1, float rx2, float ry2, float ra,
                                           float cx1, float cy1, float cx2, float cy2, float ca,
                                           float t, double mid, float pinf, float ninf) {
    if (MODE == MODE_LITERAL) {
        const float xx1 = max2(rx1, cx1, pinf);
        const float yy1 = max2(ry1, cy1, pinf);
        const float xx2 = min2(rx2, cx2, ninf);
        const float yy2 = min2(ry2, cy2, ninf);
        const float w = max2(xx2 - xx1, 0.0f, pinf);
        const float h = max2(yy2 - yy1, 0.0f, pinf);
        const float inter = w * h;
        const float uni = (ra + ca) - inter;
        return exceeds<MODE>(inter, uni, t, mid);
    }
    // The division-free modes run only on ordered boxes (x1 < x2, y1 < y2).
    // Then each column coordinate is clamped into the row box's extent,
    // med3(c, r1, r2) = min(max(c, r1), r2), and the clamped pair is ordered,
    // so w and h come out >= 0 with no clamp of their own.  Where the boxes
    // overlap in x, the clamped coordinates are max(rx1, cx1) and min(rx2,
    // cx2) themselves (cx1 <= rx2 and cx2 >= rx1 there), so w is the
    // definition's width bit for bit; where they do not, both clamp to the
    // same end of the row box and w = 0, as max(0, xx2 - xx1) gives.  The same
    // holds for h, so the intersection is the definition's in every case.
    const float inter = intersection(rx1, ry1, rx2, ry2, cx1, cy1, cx2, cy2);
    const float uni = (ra + ca) - inter;
    return exceeds<MODE>(inter, uni, t, mid);
}

struct MaskArgs {
    int n, words, mstride, npad;
    float t;
    double mid;
    int odd, exact_ok;
    float pinf, ninf;  // +inf and -inf, see max2/min2
    // Each (row tile, strip) pair is split into 1 << qshift work items of
    // 64 >> qshift rows: with few row tiles, whole pairs would leave most of
    // the GPU idle while one wave works through 64 rows.
    int qshift;
    // the sort wrote the quantised pre-test words (one image, radix passes)
    int use_packs;
    // > 0: the launch's pair count, known on the host (the one-launch path,
    // where the control block is written by the same launch); 0: read it
    // from the control block
    int items_known;
    // write dense rows (every band word) besides the lists
    int dense;
};

// Read-only inputs and the output of the mask kernel.  They are separate
// __restrict__ kernel parameters so the compiler can prove the uniform row
// loads never alias the mask stores and serve them from the scalar cache.
// Stores for data another workgroup reads while this kernel runs: device
// scope (coherent across the XCDs' L2 caches) when COHERENT.
template <bool COHERENT>
__device__ __forceinline__ void put64(uint64_t *p, uint64_t v) {
    if (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}
template <bool COHERENT>
__device__ __forceinline__ void put32(uint32_t *p, uint32_t v) {
    if (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

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
    const uint32_t *__restrict__ scol;  // coarse column words, then row words
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

// Row boxes of a work item.  Normally each row's box and area are loaded
// when the row is reached (uniform loads, which the standalone kernels serve
// from the scalar cache).  LANE_ROWS: lane k loaded row k's box and area at
// the start of the item, together with the column boxes, and each row is
// broadcast from its lane: one round trip to memory per item instead of one
// per row, for launches where the sorted boxes were written by the same
// launch and the loads cannot take the scalar path.
struct LaneRows {
    float4 box;
    float area;
};

template <bool LANE_ROWS>
__device__ __forceinline__ void row_box(const MaskPtrs &m_, int p, int k, const LaneRows &lr,
                                        float &x1, float &y1, float &x2, float &y2, float &ar) {
    if constexpr (LANE_ROWS) {
        x1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lr.box.x), k));
        y1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lr.box.y), k));
        x2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lr.box.z), k));
        y2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lr.box.w), k));
        ar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lr.area), k));
    } else {
        const float4 rb = m_.sb[p];
        x1 = rb.x;
        y1 = rb.y;
        x2 = rb.z;
        y2 = rb.w;
        ar = m_.area[p];
    }
}

// The rows k_lo .. k_hi - 1 of a work item in the division-free modes (t > 0,
// ordered boxes).  With t > 0 a pair whose intersection is exactly 0 never
// suppresses, and most pairs do not overlap, so each group of TG tiles first
// asks whether any lane may overlap in any of them, and only then are the
// tiles tested one by one; a tile where no lane may overlap is skipped, and
// words that stay 0 need no write (they start at 0).  Two forms of the
// question:
//  * SIGN: a pair can overlap only if rx2 - cx1, cx2 - rx1, ry2 - cy1 and
//    cy2 - ry1 are all >= 0 (when one is negative, the column box's clamped
//    extent in that axis is empty).  Float subtraction of finite values keeps
//    the sign of the exact difference (a tie gives +0), so the four
//    differences ORed have a clear sign bit for every pair that may overlap;
//    a tile that passes computes its intersection, union and test.  Four
//    subtractions and three ORs per pair, all of the cheap issue class.
//  * otherwise the intersections themselves, ORed (all are >= 0), and kept
//    for the tiles that pass: more work per pair but a shorter chain of
//    dependent instructions where a tile passes.
// Outside the item that holds the diagonal tile every column tile lies after
// the row's tile, and columns that take no part (tiles past the band, padding
// past n) hold an empty box at 0, whose intersection is exactly 0, so no mask
// is applied there.  In the diagonal item (DIAG) only columns after row k vote
// in the diagonal tile, and tiles before the row's tile are masked out.
template <int S, bool GROUPED, int MODE, bool DIAG, bool SIGN, bool LANE_ROWS>
__device__ __forceinline__ void fast_rows(const MaskArgs &a, const MaskPtrs &m_, int p0, int k_lo,
                                          int k_hi, const float (&cx1)[S], const float (&cy1)[S],
                                          const float (&cx2)[S], const float (&cy2)[S],
                                          const uint32_t (&cg)[S],
                                          const uint64_t (&tmask)[S], int t_diag,
                                          uint32_t (&out_lo)[S], uint32_t (&out_hi)[S],
                                          const LaneRows &lr) {
    // tiles per question: measured at 65,536 boxes, the sign form is
    // fastest asking per 2 tiles (0.357 ms; 0.368 per 4, 0.405 per 8, 0.385
    // per tile), the intersection form per 4
    constexpr int TG = SIGN ? 2 : 4;
    for (int k = k_lo; k < k_hi; ++k) {
        const int p = p0 + k;
        float rx1, ry1, rx2, ry2, ra;
        row_box<LANE_ROWS>(m_, p, k, lr, rx1, ry1, rx2, ry2, ra);
        const uint32_t rg = GROUPED ? m_.seg[p] : 0u;
        const uint64_t dmask = k == 63 ? 0ull : (~0ull << (k + 1));
#pragma unroll
        for (int t0 = 0; t0 < S; t0 += TG) {
            // SIGN: sign words of the differences; otherwise the intersections
            uint32_t sgn[TG];
            float inter[TG];
            uint32_t acc = SIGN ? ~0u : 0u;
#pragma unroll
            for (int j = 0; j < TG; ++j) {
                const int t = t0 + j;
                if (SIGN) {
                    sgn[j] = __float_as_uint(rx2 - cx1[t]) | __float_as_uint(cx2[t] - rx1) |
                             __float_as_uint(ry2 - cy1[t]) | __float_as_uint(cy2[t] - ry1);
                    acc &= sgn[j];
                } else {
                    inter[j] = intersection(rx1, ry1, rx2, ry2, cx1[t], cy1[t], cx2[t], cy2[t]);
                    acc |= __float_as_uint(inter[j]);
                }
            }
            // SIGN: the AND has a clear sign bit when some tile's OR has;
            // otherwise the OR of non-negative intersections is 0 when all are
            if (__ballot(SIGN ? (int32_t)acc >= 0 : acc != 0u) == 0ull) continue;
#pragma unroll
            for (int j = 0; j < TG; ++j) {
                const int t = t0 + j;
                uint64_t touch = __ballot(SIGN ? (int32_t)sgn[j] >= 0 : inter[j] > 0.0f);
                if (DIAG) touch &= tmask[t] & ((t == t_diag) ? dmask : ~0ull);
                if (touch) {
                    const float in =
                        SIGN ? intersection(rx1, ry1, rx2, ry2, cx1[t], cy1[t], cx2[t], cy2[t])
                             : inter[j];
                    // the column's area by the sort's expression (not held)
                    const float ca = (cx2[t] - cx1[t]) * (cy2[t] - cy1[t]);
                    const float uni = (ra + ca) - in;
                    bool pred = exceeds<MODE>(in, uni, a.t, a.mid);
                    if (GROUPED) pred = pred && (cg[t] == rg);
                    const uint64_t m = __ballot(pred) & touch;
                    out_lo[t] = write_lane(out_lo[t], (uint32_t)m, k);
                    out_hi[t] = write_lane(out_hi[t], (uint32_t)(m >> 32), k);
                }
            }
        }
    }
}

// The rows k_lo .. k_hi - 1 of a work item with the quantised pre-test
// (one image, t > 0, ordered boxes, sorted by a path that writes the coarse
// words).  The coarse question (COARSE_* in nms_internal.h): one
// subtraction per pair asks all four coordinate orders at once, and a set
// bit 7 in any byte rules the overlap out.  Each tile is asked on its own
// (an AND across tiles would not do: columns on opposite sides of the row
// clear each other's bits); the smallest of a lane's masked differences is
// 0 exactly where one of its tiles may overlap, so one ballot settles the
// row when no lane passes, as most rows do.  Only the coarse column words
// are held in registers.  For a row that passes, each tile with a passing
// lane loads its float column boxes (from the cache: every item of the
// column tile reads them) and computes the float32 intersection and
// threshold test as fast_rows() does, with the column's area recomputed by
// the sort's expression; lanes that failed the question stay out of the
// word.
template <int S, bool GROUPED, int MODE, bool DIAG>
__device__ __forceinline__ void packed_rows(const MaskArgs &a, const MaskPtrs &m_, int p0, int c0,
                                            int k_lo, int k_hi, const uint32_t (&ccw)[S],
                                            const uint64_t (&tmask)[S], int t_diag,
                                            uint32_t (&out_lo)[S], uint32_t (&out_hi)[S]) {
    static_assert(!GROUPED, "grouped input has no pre-test words");
    const int lane = threadIdx.x & 63;
    const uint32_t *__restrict__ srow = m_.scol + a.npad;
    // One row: the coarse question for its 8 tiles, then, where some lane
    // passes, the float test of the tiles that have such a lane.
    auto row = [&](int k, uint32_t rw) {
        const int p = p0 + k;
        const uint64_t dmask = k == 63 ? 0ull : (~0ull << (k + 1));
        // one question for the whole row first: the smallest of the tiles'
        // masked differences is 0 where some tile may overlap (most rows
        // have none, and cost one branch)
        uint32_t h[S];
#pragma unroll
        for (int t = 0; t < S; ++t) h[t] = (ccw[t] - rw) & COARSE_SIGNS;
        uint32_t least = h[0];
#pragma unroll
        for (int t = 1; t < S; ++t) least = least < h[t] ? least : h[t];
        if (__ballot(least == 0u) == 0ull) return;
        const float4 rb = m_.sb[p];
        const float ra = m_.area[p];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            uint64_t touch = __ballot(h[t] == 0u);
            if (DIAG) touch &= tmask[t] & ((t == t_diag) ? dmask : ~0ull);
            if (touch) {
                // columns of the tile (padding past n and tiles outside the
                // band never pass the pre-test, so their lanes stay out of
                // touch)
                const float4 cb = m_.sb[64 * (c0 + t) + lane];
                const float in = intersection(rb.x, rb.y, rb.z, rb.w, cb.x, cb.y, cb.z, cb.w);
                const float ca = (cb.z - cb.x) * (cb.w - cb.y);
                const float uni = (ra + ca) - in;
                const bool pred = exceeds<MODE>(in, uni, a.t, a.mid);
                const uint64_t m = __ballot(pred) & touch;
                out_lo[t] = write_lane(out_lo[t], (uint32_t)m, k);
                out_hi[t] = write_lane(out_hi[t], (uint32_t)(m >> 32), k);
            }
        }
    };
    // Four rows per trip, their row words in one 16-byte load (k_lo is 0:
    // the pre-test form is only used for whole row tiles).  Rows past n in
    // the last group hold COARSE_NO_ROW and never pass.
    for (int k = k_lo; k < k_hi; k += 4) {
        const uint4 r4 = *reinterpret_cast<const uint4 *>(srow + p0 + k);
        row(k, r4.x);
        row(k + 1, r4.y);
        row(k + 2, r4.z);
        row(k + 3, r4.w);
    }
}

// Fused launch: report a finished item of row tile `pending` (if any) by
// adding to done[pending].  The data the sweep reads was written with
// device-scope stores, which write through the XCD's L2; once they are
// acknowledged (s_waitcnt vmcnt(0) also counts stores) they are visible to
// device-scope loads on every XCD, so a reader that sees the count sees the
// data.  No L2 write-back (a release fence) is needed: that is for plain
// stores, and the sweep reads none of those.  Every lane adds 1, so a
// finished pair counts 64 << qshift: a lane-0-only branch here would put a
// lane-divergent region in the caller's loop.
// (The row tile is made visibly uniform: with an address the compiler takes
// for a per-lane one, the 64 lanes' additions go out as 64 atomics instead
// of one.)
__device__ __forceinline__ void report_done(uint32_t *done, int &pending) {
    const int r = __builtin_amdgcn_readfirstlane(pending);
    if (r < 0) return;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
    __hip_atomic_fetch_add(&done[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pending = -1;
}

// One work item.  COHERENT (the fused mask + sweep kernel): the near words
// and list entries, which the sweep reads while other items are still
// running, are written with device-scope stores, and once they have all
// completed the item adds 64 to done[r] (one per lane), the count of
// finished items of its row tile times 64.  Plain stores may sit in the L2 of this XCD, which the sweep's
// XCD does not see.
template <int S, bool GROUPED, int MODE, bool COHERENT, bool PACKED, bool LANE_ROWS = false>
__device__ __forceinline__ void mask_item(const MaskArgs &a, const MaskPtrs &m_, int item,
                                          int stride, uint32_t *done, int &pending) {
    const int lane = threadIdx.x & 63;
    // the item's pair and rows within it
    const int rpi = 64 >> a.qshift;
    const int pair = item >> a.qshift;
    const int k_lo = (item & ((1 << a.qshift) - 1)) * rpi;
    // Row tile of this pair: the largest r whose first pair is <= pair.  One
    // image: every row tile covers all strips from its own to the last, so
    // the first pair of row tile r has a closed form (a triangle of strips)
    // and the search is register arithmetic; grouped input searches the
    // plan's table.
    int lo = 0, hi = a.words - 1;
    int32_t base_r;
    if (!GROUPED) {
        const int G = (a.words + S - 1) / S;
        auto first_pair = [&](int rr) {
            const int g = rr / S, u = rr % S;
            return S * (g * G - g * (g - 1) / 2) + u * (G - g);
        };
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first_pair(mid) <= pair) lo = mid;
            else hi = mid - 1;
        }
        base_r = first_pair(lo);
    } else {
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (m_.item_base[mid] <= pair) lo = mid;
            else hi = mid - 1;
        }
        base_r = m_.item_base[lo];
    }
    const int r = lo;
    const int s0 = r / S;
    const int c0 = (s0 + (pair - base_r)) * S;
    const int cend = m_.tile_cend[r];
    const int p0 = 64 * r;
    const int tile_rows = a.n - p0 < 64 ? a.n - p0 : 64;
    const int k_hi = k_lo + rpi < tile_rows ? k_lo + rpi : tile_rows;
    // lanes k_lo .. k_hi - 1 end up holding the words of rows k_lo .. k_hi - 1
    const bool mine = lane >= k_lo && lane < k_hi;
    const int t_diag = r - c0;  // the diagonal tile's slot, if it lies in this strip

    // Column boxes of the strip, one per lane and tile.  Tiles outside
    // [r, cend) are evaluated and masked out (tmask = 0), which costs less
    // than branching around them; their boxes are replaced by an empty box
    // at 0, whose intersection with anything is exactly 0 (like the padding
    // boxes past n), so they never look like an overlap.
    // With the quantised pre-test the columns' coarse pre-test words take the
    // place of the boxes.
    static_assert(!PACKED || (!GROUPED && MODE != MODE_LITERAL), "pre-test words: one image");
    float cx1[S], cy1[S], cx2[S], cy2[S];
    uint32_t cg[S], clo[S];
    uint64_t tmask[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
        const int c = c0 + t;
        const bool active = c >= r && c < cend;
        const int q = active ? 64 * c + lane : lane;
        if constexpr (PACKED) {
            // the coarse column words (the float boxes are loaded where a
            // row passes)
            clo[t] = active ? m_.scol[q] : COARSE_NONE;
        } else {
            const float4 b = active ? m_.sb[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            cx1[t] = b.x;
            cy1[t] = b.y;
            cx2[t] = b.z;
            cy2[t] = b.w;
        }
        if (GROUPED) cg[t] = m_.seg[q];
        tmask[t] = active ? column_valid(c, a.n) : 0ull;
    }
    LaneRows lr;
    if constexpr (LANE_ROWS) {
        static_assert(!PACKED, "lane rows: the float form only");
        lr.box = m_.sb[p0 + lane];   // rows past n are the zero padding
        lr.area = m_.area[p0 + lane];
    }
    uint32_t out_lo[S], out_hi[S];
#pragma unroll
    for (int t = 0; t < S; ++t) out_lo[t] = out_hi[t] = 0u;

    if (MODE == MODE_LITERAL) {
        for (int k = k_lo; k < k_hi; ++k) {
            const int p = p0 + k;
            float rx1, ry1, rx2, ry2, ra;
            row_box<LANE_ROWS>(m_, p, k, lr, rx1, ry1, rx2, ry2, ra);
            const uint32_t rg = GROUPED ? m_.seg[p] : 0u;
            // in the diagonal tile only boxes after row k vote
            const uint64_t dmask = k == 63 ? 0ull : (~0ull << (k + 1));
#pragma unroll
            for (int t = 0; t < S; ++t) {
                const uint64_t live = tmask[t] & ((t == t_diag) ? dmask : ~0ull);
                bool pred = suppresses<MODE>(rx1, ry1, rx2, ry2, ra, cx1[t], cy1[t], cx2[t],
                                             cy2[t], (cx2[t] - cx1[t]) * (cy2[t] - cy1[t]),
                                             a.t, a.mid, a.pinf, a.ninf);
                if (GROUPED) pred = pred && (cg[t] == rg);
                const uint64_t m = __ballot(pred) & live;
                out_lo[t] = write_lane(out_lo[t], (uint32_t)m, k);
                out_hi[t] = write_lane(out_hi[t], (uint32_t)(m >> 32), k);
            }
        }
    } else {
        // Few work items (qshift > 0) leave the GPU mostly idle and the item's
        // latency decides: the intersections come first, as the pass test
        // needs them anyway.  With many items the issue rate decides, and the
        // sign test costs fewer and cheaper instructions.
        const bool diag = t_diag >= 0 && t_diag < S;
        if constexpr (PACKED) {
            {
                if (diag)
                    packed_rows<S, GROUPED, MODE, true>(a, m_, p0, c0, k_lo, k_hi, clo,
                                                        tmask, t_diag, out_lo, out_hi);
                else
                    packed_rows<S, GROUPED, MODE, false>(a, m_, p0, c0, k_lo, k_hi, clo,
                                                         tmask, t_diag, out_lo, out_hi);
            }
        }
        if constexpr (PACKED) {
        } else if (a.qshift == 0) {
            if (diag)
                fast_rows<S, GROUPED, MODE, true, true, LANE_ROWS>(a, m_, p0, k_lo, k_hi, cx1, cy1, cx2,
                                                                   cy2, cg, tmask, t_diag, out_lo,
                                                                   out_hi, lr);
            else
                fast_rows<S, GROUPED, MODE, false, true, LANE_ROWS>(a, m_, p0, k_lo, k_hi, cx1, cy1, cx2,
                                                                    cy2, cg, tmask, t_diag, out_lo,
                                                                    out_hi, lr);
        } else {
            if (diag)
                fast_rows<S, GROUPED, MODE, true, false, LANE_ROWS>(a, m_, p0, k_lo, k_hi, cx1, cy1, cx2,
                                                                    cy2, cg, tmask, t_diag, out_lo,
                                                                    out_hi, lr);
            else
                fast_rows<S, GROUPED, MODE, false, false, LANE_ROWS>(a, m_, p0, k_lo, k_hi, cx1, cy1,
                                                                     cx2, cy2, cg, tmask, t_diag,
                                                                     out_lo, out_hi, lr);
        }
    }
    // COHERENT: the previous item's count, once its stores are acknowledged
    // (they have had this item's computation to complete)
    if (COHERENT) report_done(done, pending);
    if (mine) {
        const int p = p0 + lane;
        if (a.dense) {
            uint64_t *dst = m_.mask + (size_t)p * (size_t)stride + (size_t)(c0 - s0 * S);
            uint4 *d4 = reinterpret_cast<uint4 *>(dst);
#pragma unroll
            for (int t = 0; t < S; t += 2)
                d4[t / 2] = make_uint4(out_lo[t], out_hi[t], out_lo[t + 1], out_hi[t + 1]);
        }
        // transposed copies of the words for tiles r .. r + NEAR_TILES
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const int j = t - t_diag;
            if (j >= 0 && j <= NEAR_TILES && c0 + t < cend)
                put64<COHERENT>(&m_.tnear[(size_t)j * a.npad + p],
                                ((uint64_t)out_hi[t] << 32) | out_lo[t]);
        }
    }
    // Record the strip's nonzero words in the row tile's list.  A wave-wide
    // prefix sum gives each lane its place and one atomic claims the wave's
    // slots, so the list order may differ from run to run; the sweep only ORs
    // entries together, which does not depend on their order.  Entries past
    // the capacity are dropped and the count (which still grows) tells the
    // sweep to read dense rows instead.
    uint32_t nz = 0;
    if (mine) {
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
            if ((out_lo[t] | out_hi[t]) != 0u && mine) {
                if (at < (uint32_t)TILE_LIST_CAP) {
                    const size_t e = (size_t)r * TILE_LIST_CAP + at;
                    put32<COHERENT>(&m_.tent_wk[e], ((uint32_t)(c0 + t) << 6) | (uint32_t)lane);
                    put64<COHERENT>(&m_.tent_val[e], ((uint64_t)out_hi[t] << 32) | out_lo[t]);
                }
                ++at;
            }
        }
    }
    // the count is reported with the next item's stores, or after the loop
    if (COHERENT) pending = r;
}

// The work items of one launch, handed out to waves in item order (row tile
// by row tile): wave slot `first` of `slots` takes items first, first +
// slots, ... (launches give every wave at most one item unless the item
// count exceeds what a grid can hold)
//
// PACKED_ONLY (the fused launch, which runs for one image of at least 512
// row tiles, always radix-sorted and never split): the division-free modes
// come only in the pre-test form, so the kernel holds no code, and reserves
// no registers, for the other forms.
//
// queue (the fused launch): the workgroup owns the block of `slots` items
// from `first` on, and each of its waves takes the block's next item from a
// counter in LDS until none is left.  A workgroup's waves keep taking items
// while one of them is still busy, where with one item per wave the
// workgroup (eight waves) would hold its slot until its slowest wave ended.
// Blocks start in workgroup order, so items still finish row tile by row
// tile.  (One counter in device memory for all waves was tried: its atomics
// serialise, and the launch took twice as long.)
template <int S, bool GROUPED, bool COHERENT, bool PACKED_ONLY = false, bool LANE_ROWS = false>
__device__ __forceinline__ void mask_items(const MaskArgs &a, const MaskPtrs &m_,
                                           const Ctrl *__restrict__ ctrl, int first, int slots,
                                           uint32_t *done, uint32_t *queue = nullptr) {
    static_assert(!(PACKED_ONLY && GROUPED), "grouped input has no pre-test words");
    const int num_items = (a.items_known > 0 ? a.items_known : ctrl->num_items) << a.qshift;
    const bool fast = (ctrl->flags & FLAG_ORDERED_BOXES) && a.exact_ok;
    const bool packed = a.use_packs && a.qshift == 0;
    const int stride = GROUPED ? ctrl->band_stride : a.mstride;
    // queue: a counter in LDS over the workgroup's block of `slots` items
    // from `first` on
    const int end = queue ? (first + slots < num_items ? first + slots : num_items) : num_items;
    auto next_item = [&](int item) -> int {
        if (queue == nullptr) return item + slots;
        uint32_t got = 0;
        if ((threadIdx.x & 63) == 0)
            got = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return first + (int)__builtin_amdgcn_readfirstlane(got);
    };
    int pending = -1;  // COHERENT: row tile of a finished item not yet counted
    for (int item = queue ? next_item(0) : first; item < end; item = next_item(item)) {
        if (fast) {
            if constexpr (!GROUPED) {
                if (PACKED_ONLY || packed) {
                    if (a.odd) mask_item<S, false, MODE_ODD, COHERENT, true>(a, m_, item, stride, done, pending);
                    else mask_item<S, false, MODE_EVEN, COHERENT, true>(a, m_, item, stride, done, pending);
                    continue;
                }
            }
            if constexpr (!PACKED_ONLY) {
                if (a.odd)
                    mask_item<S, GROUPED, MODE_ODD, COHERENT, false, LANE_ROWS>(a, m_, item, stride,
                                                                                done, pending);
                else
                    mask_item<S, GROUPED, MODE_EVEN, COHERENT, false, LANE_ROWS>(a, m_, item, stride,
                                                                                 done, pending);
            }
        } else {
            mask_item<S, GROUPED, MODE_LITERAL, COHERENT, false, LANE_ROWS>(a, m_, item, stride, done,
                                                                            pending);
        }
    }
    if (COHERENT) report_done(done, pending);
}

// Kernel arguments of the mask stage, filled on the host; `slots` is the
// number of waves that take work items at once.
MaskArgs make_mask_args(const Problem &P, const Layout &L, int64_t slots);
// Upper bound on the work items of a launch (every row tile covers all
// strips to the end).
int64_t mask_items_upper_bound(const Problem &P, const Layout &L);

}  // namespace maskcore
}  // namespace gnms
