// Stage (b): the triangle-tiled IoU suppression bitmask.
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
// expression "inter / union > t".  When every box is ordered (x1 < x2, y1 <
// y2) with a finite area > 0 (checked by the last sort pass, which gathers
// the boxes), 0 <= inter <= union and union > 0, and
// the test is exactly equivalent to comparing inter against m * union in
// binary64, where m = t + ulp(t)/2 is the rounding boundary above t: the
// product of a 25-bit m and a 24-bit union is exact in binary64, and the
// float32 quotient exceeds t iff the real quotient reaches m (ties at m round
// up when t's last significand bit is odd, to t when it is even).  That costs
// two conversions, one multiply and one compare instead of a correctly
// rounded division; the intersection then takes 4 clamps, 2 subtractions
// and a multiply (see suppresses()), 13 vector instructions per 64 pairs in
// all.  Otherwise (degenerate or inverted boxes, t <= 0) the kernel performs
// the literal float32 division.
#include <cmath>
#include <cstring>

#include "mask_core.h"
#include "nms_internal.h"

#pragma clang fp contract(off)

namespace gnms {
namespace {

using namespace maskcore;

// ---------------------------------------------------------------- mask

template <int S, bool GROUPED>
// (4 waves per SIMD: at most 128 registers)
__global__ __launch_bounds__(MASK_THREADS, 4) void mask_kernel(
    MaskArgs a, const Ctrl *__restrict__ ctrl, const float4 *__restrict__ sb,
    const float *__restrict__ area, const uint32_t *__restrict__ seg,
    const int32_t *__restrict__ tile_cend, const int32_t *__restrict__ item_base,
    uint64_t *__restrict__ mask, uint32_t *__restrict__ tcount, uint32_t *__restrict__ tent_wk,
    uint64_t *__restrict__ tent_val, uint64_t *__restrict__ tnear,
    const uint32_t *__restrict__ scol) {
    const MaskPtrs m_{sb,     area,    seg,      tile_cend, item_base,
                      mask,   tcount,  tent_wk,  tent_val,  tnear,     scol};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves_per_block = MASK_THREADS / 64;
    mask_items<S, GROUPED, false>(a, m_, ctrl, blockIdx.x * waves_per_block + wave,
                                  gridDim.x * waves_per_block, nullptr);
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

}  // namespace

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

namespace maskcore {

MaskArgs make_mask_args(const Problem &P, const Layout &L, int64_t slots) {
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
    // Too few pairs to give every slot one: split them into up to 16 groups
    // of rows while the items still fit the resident waves.  An item costs
    // a few memory round trips whatever its rows, and items of one row tile
    // share its list's counter, so items past the slots cost more than they
    // save.  Grouped input has short bands, and the bound here counts full
    // rows, so its pairs are always split.
    const int64_t pairs = mask_items_upper_bound(P, L);
    a.qshift = 0;
    while (a.qshift < 4 && (pairs << (a.qshift + 1)) <= slots) ++a.qshift;
    if (P.grouped) a.qshift = 2;
    // the radix sort of one image writes the quantised pre-test words
    a.use_packs = (!P.grouped && P.n > RANK_SORT_MAX) ? 1 : 0;
    a.items_known = 0;
    a.dense = P.dense ? 1 : 0;
    return a;
}

int64_t mask_items_upper_bound(const Problem &P, const Layout &L) {
    const int64_t W = L.words;
    const int S = P.strip;
    int64_t items_ub = 0;
    for (int64_t r = 0; r < W; r += S) {
        const int64_t rows_here = (r + S <= W) ? S : (W - r);
        items_ub += rows_here * ((W + S - 1) / S - r / S);
    }
    return items_ub;
}

}  // namespace maskcore

// Slots that the split of small inputs aims at: 16 waves per CU.  The
// kernel's registers allow 6 waves per SIMD (24 per CU), but splitting for 24
// cost the clustered 8192-box case 4.5 us (0.033 -> 0.037 ms) and gained 4096
// boxes 1 us; splitting for 8 cost both (0.049, 0.021 ms).
static maskcore::MaskArgs separate_mask_args(const Problem &P, const Layout &L) {
    const int64_t slots = (int64_t)device_cu_count() * 16;
    return maskcore::make_mask_args(P, L, slots);
}

int separate_mask_qshift(const Problem &P, const Layout &L) {
    return separate_mask_args(P, L).qshift;
}

hipError_t launch_mask(const Problem &P, const Layout &L, const Work &w, hipStream_t stream) {
    const int waves_per_block = MASK_THREADS / 64;
    const maskcore::MaskArgs a = separate_mask_args(P, L);
    const int64_t items_ub = maskcore::mask_items_upper_bound(P, L) << a.qshift;
    // one work item per wave: the GPU starts workgroups as earlier ones
    // leave, which evens out waves that progress at different rates
    int64_t blocks = (items_ub + waves_per_block - 1) / waves_per_block;
    if (blocks > MAX_GRID_THREADS / MASK_THREADS) blocks = MAX_GRID_THREADS / MASK_THREADS;
    if (blocks < 1) blocks = 1;
    if (P.grouped)
        hipLaunchKernelGGL((mask_kernel<STRIP_GROUPED, true>), dim3((unsigned)blocks),
                           dim3(MASK_THREADS), 0, stream, a, w.ctrl, w.sb, w.area, w.seg,
                           w.tile_cend, w.item_base, w.mask, w.tcount, w.tent_wk, w.tent_val,
                           w.tnear, w.scol);
    else
        hipLaunchKernelGGL((mask_kernel<STRIP_SINGLE, false>), dim3((unsigned)blocks),
                           dim3(MASK_THREADS), 0, stream, a, w.ctrl, w.sb, w.area, w.seg,
                           w.tile_cend, w.item_base, w.mask, w.tcount, w.tent_wk, w.tent_val,
                           w.tnear, w.scol);
    return hipGetLastError();
}

hipError_t launch_decide(const float *inter, const float *uni, int64_t count, float thresh,
                         bool positive_areas, uint8_t *out, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const Threshold th = make_threshold(thresh);
    int mode = maskcore::MODE_LITERAL;
    if (positive_areas && th.exact_ok) mode = th.odd ? maskcore::MODE_ODD : maskcore::MODE_EVEN;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(decide_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, inter, uni,
                       count, thresh, th.mid, mode, out);
    return hipGetLastError();
}

}  // namespace gnms
