// Helpers shared by the sort kernels (radix.hip, team_sort.hip): the sort
// keys, wave-wide scans, and the quantised pre-test words of a sorted box.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nms_internal.h"

namespace gnms {
namespace sortcore {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Inclusive sum over the lanes of the wave, in DPP steps (no LDS round
// trips): shifts by 1, 2, 4 and 8 lanes within each row of 16 (a lane shifted
// in from outside the row adds 0), then row 0's total into row 1 and row
// 2's into row 3 (lane 15's broadcast), then rows 0 and 1's into rows 2 and
// 3 (lane 31's).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~asc;
}

// signed class id -> unsigned key with the same order
__device__ __forceinline__ uint32_t class_key(int32_t c) { return (uint32_t)c ^ 0x80000000u; }

// Image of input box i: the largest m < num_images with off[m] <= i.
__device__ __forceinline__ uint32_t image_of(const int64_t *off, int num_images, int64_t i) {
    int lo = 0, hi = num_images - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    return (uint32_t)lo;
}

// Lanes add into HIST_COPIES interleaved copies of the histograms: keys of
// real scores share their top digits (the float exponent), and atomics of
// many lanes on one LDS word serialise.
constexpr int HIST_COPIES = 4;

// Exclusive scan of v[0..256) into out[] by one wave (4 per lane).
__device__ __forceinline__ void scan256(const uint32_t *v, uint32_t *out) {
    const int lane = lane_id();
    const uint32_t h0 = v[4 * lane], h1 = v[4 * lane + 1], h2 = v[4 * lane + 2],
                   h3 = v[4 * lane + 3];
    const uint32_t s = h0 + h1 + h2 + h3;
    const uint32_t ex = wave_incl_sum(s) - s;
    out[4 * lane] = ex;
    out[4 * lane + 1] = ex + h0;
    out[4 * lane + 2] = ex + h0 + h1;
    out[4 * lane + 3] = ex + h0 + h1 + h2;
}

// The grid of the quantised pre-test (see PACK_QMAX in nms_internal.h):
// q(v) = min(floor((v - lo) * s), QMAX - 1), which never reverses an order.
struct PackScale {
    float x0, y0, sx, sy;
};

__device__ __forceinline__ uint32_t quantise(float v, float lo, float s) {
    const float q = fminf(fmaxf(floorf((v - lo) * s), 0.0f), (float)(PACK_QMAX - 1u));
    return (uint32_t)q;
}

__device__ __forceinline__ uint32_t coarse(uint32_t q) { return min(q >> 8, 126u); }

// The coarse words (col, row) of one box (see PACK_QMAX and COARSE_* in
// nms_internal.h).
__device__ __forceinline__ uint2 coarse_words(float4 b, const PackScale &ps) {
    const uint32_t vx1 = coarse(quantise(b.x, ps.x0, ps.sx));
    const uint32_t vy1 = coarse(quantise(b.y, ps.y0, ps.sy));
    const uint32_t vx2 = coarse(quantise(b.z, ps.x0, ps.sx));
    const uint32_t vy2 = coarse(quantise(b.w, ps.y0, ps.sy));
    return make_uint2((0xFFu - vx2) | (0x7Fu + vx1) << 8 | (0xFFu - vy2) << 16 | (0x7Fu + vy1) << 24,
                      (0x80u - vx1) | vx2 << 8 | (0x80u - vy1) << 16 | vy2 << 24);
}

// Grid step for an axis of extent lo .. hi: QMAX - 1 steps, or 0 (every
// coordinate on step 0, so the pre-test rules nothing out) when the extent
// is empty, not finite or too small for a finite step.
__device__ __forceinline__ float pack_step(float lo, float hi) {
    const float d = hi - lo;
    if (!(d > 0.0f) || !(d < INFINITY)) return 0.0f;
    const float s = (float)(PACK_QMAX - 1u) / d;
    return s < INFINITY ? s : 0.0f;
}

}  // namespace sortcore
}  // namespace gnms
