// Stages (c) and (d): the greedy sweep over the suppression bitmask, then the
// compaction that maps kept sorted positions back to input indices.
//
// Sweep ("LeetCUDA 14-nms", Phase 2).  One workgroup keeps the removed bitmap
// (one bit per sorted box, W = ceil(n/64) words) in LDS and visits the boxes
// in score order.  The page takes one barrier per box; here the boxes go in
// chunks of 64 (one row tile), with one barrier per chunk between resolving
// and propagating:
//   * resolve: wave 0 loads the 64 diagonal words M[64c + k][c] (one per
//     lane) and settles the chunk serially in scalar registers: the lowest
//     not-yet-removed row k whose diagonal word is nonzero is kept and its
//     word is ORed into the chunk's removed word; rows whose diagonal word is
//     zero cannot remove anything inside the chunk, so only rows that both
//     survive and suppress cost a step.  Every row still clear at the end is
//     kept.  A row's word only has bits above the row, so a later step never
//     changes an earlier decision.
//   * propagate: all 1024 threads OR the kept rows' words for the column
//     tiles after the chunk (up to the end of the row tile's band) into the
//     LDS bitmap; thread j owns word c + 1 + j, so no atomics are needed.
// A box is kept iff its removed bit is clear when the sweep reaches it, and
// later rows never set bits at or below their own position, so the kept set
// is the complement of the final bitmap.
//
// Compaction (the page's host-side map-back, bug 3, done on the device).  For
// one image the sorted order is the score order: kept bits are counted per
// word, prefix-summed across the workgroup and written as int64 input
// indices order[p].  For grouped input the kept bits are in group order; the
// compaction kernel walks the plain score order and looks each box's sorted
// position up through the inverse permutation, so the output is one list in
// global score order.
#include "nms_internal.h"

namespace gnms {
namespace {

constexpr int NT = SWEEP_THREADS;
constexpr int NWAVES = NT / 64;

struct SweepArgs {
    const uint64_t *mask;
    const int32_t *tile_cend;
    const int32_t *order;
    Ctrl *ctrl;
    uint64_t *kept;
    int64_t *keep_out;
    int n, words, mstride, strip, grouped;
};

__device__ __forceinline__ uint64_t rows_valid(int c, int n) {
    const int rem = n - 64 * c;
    return rem >= 64 ? ~0ull : ((1ull << rem) - 1ull);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t read_lane64(uint64_t v, int k) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, k);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), k);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// exclusive block prefix sum; *total receives the block sum
__device__ uint32_t block_excl_sum(uint32_t v, uint32_t *part, uint32_t *part2, uint32_t *tot,
                                   uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_sum(v);
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t s = lane < NWAVES ? part[lane] : 0u;
        const uint32_t si = wave_incl_sum(s);
        if (lane < NWAVES) part2[lane] = si - s;
        if (lane == NWAVES - 1) *tot = si;
    }
    __syncthreads();
    const uint32_t r = part2[wave] + incl - v;
    *total = *tot;
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(NT) void sweep_kernel(SweepArgs a) {
    extern __shared__ uint64_t removed[];
    __shared__ uint64_t sh_kept;
    __shared__ uint32_t part[NWAVES], part2[NWAVES], tot;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int W = a.words, n = a.n, S = a.strip;
    const int stride = a.grouped ? a.ctrl->band_stride : a.mstride;

    for (int w = tid; w < W; w += NT) removed[w] = 0ull;
    __syncthreads();

    for (int c = 0; c < W; ++c) {
        const size_t col0 = (size_t)((c / S) * S);  // first word stored for row tile c
        if (wave == 0) {
            const int p = 64 * c + lane;
            const uint64_t d = p < n ? a.mask[(size_t)p * stride + ((size_t)c - col0)] : 0ull;
            const uint64_t valid = rows_valid(c, n);
            const uint64_t nz = __ballot(d != 0ull);
            uint64_t rem = uniform64(removed[c]);
            uint64_t cand = ~rem & nz & valid;
            while (cand) {
                const int k = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cand));
                rem |= read_lane64(d, k);
                const uint64_t above = k == 63 ? 0ull : (~0ull << (k + 1));
                cand = ~rem & nz & valid & above;
            }
            if (lane == 0) {
                removed[c] = rem;
                sh_kept = ~rem & valid;
            }
        }
        __syncthreads();
        const uint64_t kept = sh_kept;
        if (kept) {
            const int cend = a.tile_cend[c];
            for (int w = c + 1 + tid; w < cend; w += NT) {
                uint64_t acc = 0ull;
                uint64_t kk = kept;
                while (kk) {
                    const int k = __builtin_ctzll(kk);
                    kk &= kk - 1ull;
                    acc |= a.mask[(size_t)(64 * c + k) * stride + ((size_t)w - col0)];
                }
                if (acc) removed[w] |= acc;
            }
        }
        __syncthreads();
    }

    // kept bitmap = complement of removed, limited to existing boxes
    for (int w = tid; w < W; w += NT) a.kept[w] = ~removed[w] & rows_valid(w, n);
    if (a.grouped) return;

    // one image: compact in sorted (= score) order, mapping back through order[]
    const int chunk = (W + NT - 1) / NT;
    const int lo = tid * chunk < W ? tid * chunk : W;
    const int hi = lo + chunk < W ? lo + chunk : W;
    uint32_t cnt = 0;
    for (int w = lo; w < hi; ++w) cnt += (uint32_t)__popcll(~removed[w] & rows_valid(w, n));
    uint32_t total = 0;
    uint32_t pos = block_excl_sum(cnt, part, part2, &tot, &total);
    for (int w = lo; w < hi; ++w) {
        uint64_t bits = ~removed[w] & rows_valid(w, n);
        while (bits) {
            const int k = __builtin_ctzll(bits);
            bits &= bits - 1ull;
            a.keep_out[pos++] = (int64_t)a.order[64 * w + k];
        }
    }
    if (tid == 0) a.ctrl->count = (int32_t)total;
}

struct CompactArgs {
    const int32_t *score_order;
    const int32_t *inv;
    const uint64_t *kept;
    Ctrl *ctrl;
    int64_t *keep_out;
    int n;
};

__global__ __launch_bounds__(NT) void compact_kernel(CompactArgs a) {
    __shared__ uint32_t part[NWAVES], part2[NWAVES], tot;
    const int tid = threadIdx.x;
    const int n = a.n;
    const int chunk = (n + NT - 1) / NT;
    const int lo = tid * chunk < n ? tid * chunk : n;
    const int hi = lo + chunk < n ? lo + chunk : n;
    uint32_t cnt = 0;
    for (int r = lo; r < hi; ++r) {
        const int p = a.inv[a.score_order[r]];
        cnt += (uint32_t)((a.kept[p >> 6] >> (p & 63)) & 1ull);
    }
    uint32_t total = 0;
    uint32_t pos = block_excl_sum(cnt, part, part2, &tot, &total);
    for (int r = lo; r < hi; ++r) {
        const int i = a.score_order[r];
        const int p = a.inv[i];
        if ((a.kept[p >> 6] >> (p & 63)) & 1ull) a.keep_out[pos++] = (int64_t)i;
    }
    if (tid == 0) a.ctrl->count = (int32_t)total;
}

// Dense copy of the mask for tests: out[p][c] for all c < W.
__global__ void expand_kernel(const uint64_t *mask, const int32_t *tile_cend, const Ctrl *ctrl,
                              uint64_t *out, int n, int words, int mstride, int strip,
                              int grouped) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n * words) return;
    const int p = (int)(idx / words);
    const int c = (int)(idx % words);
    const int r = p >> 6;
    const int stride = grouped ? ctrl->band_stride : mstride;
    const int col0 = (r / strip) * strip;
    uint64_t v = 0ull;
    if (c >= r && c < tile_cend[r]) v = mask[(size_t)p * stride + (size_t)(c - col0)];
    out[idx] = v;
}

}  // namespace

hipError_t launch_sweep(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                        hipStream_t stream) {
    SweepArgs a;
    a.mask = w.mask;
    a.tile_cend = w.tile_cend;
    a.order = w.order;
    a.ctrl = w.ctrl;
    a.kept = w.kept;
    a.keep_out = keep_out;
    a.n = P.n;
    a.words = (int)L.words;
    a.mstride = (int)L.mstride;
    a.strip = P.strip;
    a.grouped = P.grouped ? 1 : 0;
    const size_t lds = (size_t)L.words * sizeof(uint64_t);
    hipLaunchKernelGGL(sweep_kernel, dim3(1), dim3(NT), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_compact(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                          hipStream_t stream) {
    (void)L;
    CompactArgs a;
    a.score_order = w.score_order;
    a.inv = w.inv;
    a.kept = w.kept;
    a.ctrl = w.ctrl;
    a.keep_out = keep_out;
    a.n = P.n;
    hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_expand_mask(const Problem &P, const Layout &L, const Work &w,
                              uint64_t *mask_out, hipStream_t stream) {
    const int64_t total = (int64_t)P.n * L.words;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(expand_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w.mask,
                       w.tile_cend, w.ctrl, mask_out, P.n, (int)L.words, (int)L.mstride,
                       P.strip, P.grouped ? 1 : 0);
    return hipGetLastError();
}

}  // namespace gnms
