// Stage (a): score keys, stable LSD radix sort and the mask work plan.
//
// One workgroup of 1024 threads sorts all n boxes.  Greedy NMS visits boxes
// by score, highest first, with equal scores in input order ("LeetCUDA
// 14-nms", algorithm and data flow, step 1: a stable sort).  Each score maps
// to a 32-bit key whose ascending order is descending score (-0.0 is folded
// onto +0.0 so the two tie); LSD radix passes over 8-bit digits are stable,
// and the array starts in input order, so equal keys keep ascending index
// without the index taking part in any pass.
//
// Grouped input (class ids and/or several images) then gets further stable
// passes on the class id and on the image index: boxes of one (image, class)
// group become contiguous, each group still in score order.  The same kernel
// derives the per-row-tile band of column tiles the mask kernel must cover
// and the list of mask work items.
//
// A pass whose digit is equal for every key moves nothing and is skipped.
// One workgroup is enough: the sort moves O(n) bytes while the IoU mask that
// follows does O(n^2) work, and a single workgroup needs no inter-workgroup
// synchronisation and one launch.
#include "nms_internal.h"

namespace gnms {
namespace {

constexpr int NT = SORT_THREADS;
constexpr int NWAVES = NT / 64;

// Elements per thread per scatter tile.  Element i of a tile sits at
// (wave, e, lane) with i = wave * 64 * E + e * 64 + lane, so walking waves,
// then e, then lanes is walking indices in order, which keeps the pass stable.
constexpr int E = 8;
constexpr int TILE = NT * E;

struct SortSmem {
    uint32_t hist4[4][256];
    uint32_t base[256];     // next global position of each digit
    uint32_t tcnt[256];     // digit counts of the current tile
    uint32_t tbase[256];    // start of each digit's run inside the staged tile
    int32_t gsh[256];       // global position minus staged slot, per digit
    uint32_t wcnt[NWAVES][256];
    uint32_t wpre[NWAVES][256];
    uint32_t stage_k[TILE];  // one tile, reordered by digit, before it is written
    uint32_t stage_v[TILE];
    uint32_t part[NWAVES];
    uint32_t part2[NWAVES];
    uint32_t rev[NT];
    uint32_t flag;
    uint32_t err;
};

struct SortArgs {
    const float *scores;
    const int32_t *class_ids;
    const int64_t *offsets;
    int n;
    int num_images;
    int grouped;
    int words;       // W
    int npad;
    int strip;
    Work w;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v = v > u ? v : u;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_incl_min(uint32_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v = v < u ? v : u;
    }
    return v;
}

// Exclusive block-wide prefix sum of one value per thread; *total receives
// the sum over the block.  Ends with a barrier so the scratch can be reused.
__device__ uint32_t block_excl_sum(uint32_t v, SortSmem &sm, uint32_t *total) {
    const int lane = lane_id(), wave = wave_id();
    uint32_t incl = wave_incl_sum(v);
    if (lane == 63) sm.part[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint32_t s = lane < NWAVES ? sm.part[lane] : 0u;
        uint32_t si = wave_incl_sum(s);
        if (lane < NWAVES) sm.part2[lane] = si - s;
        if (lane == NWAVES - 1) sm.flag = si;
    }
    __syncthreads();
    uint32_t r = sm.part2[wave] + incl - v;
    *total = sm.flag;
    __syncthreads();
    return r;
}

// Block-wide maximum.
__device__ uint32_t block_max(uint32_t v, SortSmem &sm) {
    const int lane = lane_id(), wave = wave_id();
    uint32_t m = wave_incl_max(v);
    if (lane == 63) sm.part[wave] = m;
    __syncthreads();
    if (wave == 0) {
        uint32_t s = lane < NWAVES ? sm.part[lane] : 0u;
        s = wave_incl_max(s);
        if (lane == 63) sm.flag = s;
    }
    __syncthreads();
    uint32_t r = sm.flag;
    __syncthreads();
    return r;
}

// For each thread t: the minimum of v over threads t' > t (0xFFFFFFFF if none).
__device__ uint32_t block_suffix_min_after(uint32_t v, SortSmem &sm) {
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    sm.rev[NT - 1 - tid] = v;
    __syncthreads();
    uint32_t x = sm.rev[tid];              // logical position tid = thread NT-1-tid
    uint32_t incl = wave_incl_min(x);
    if (lane == 63) sm.part[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint32_t s = lane < NWAVES ? sm.part[lane] : 0xFFFFFFFFu;
        uint32_t si = wave_incl_min(s);
        // exclusive: min over earlier waves
        uint32_t prev = __shfl_up(si, 1, 64);
        if (lane < NWAVES) sm.part2[lane] = lane == 0 ? 0xFFFFFFFFu : prev;
    }
    __syncthreads();
    // exclusive min over logical positions < tid
    uint32_t before = __shfl_up(incl, 1, 64);
    if (lane == 0) before = 0xFFFFFFFFu;
    uint32_t ex = sm.part2[wave];
    ex = ex < before ? ex : before;
    __syncthreads();
    sm.rev[NT - 1 - tid] = ex;             // back to thread order
    __syncthreads();
    uint32_t r = sm.rev[tid];
    __syncthreads();
    return r;
}

// Histograms of all four 8-bit digits of ks[0..n) (the digit counts do not
// depend on the order the keys are in, so one read serves four passes).
__device__ void digit_histograms(const uint32_t *ks, int n, SortSmem &sm) {
    const int tid = threadIdx.x;
    uint32_t *h = &sm.hist4[0][0];
    for (int j = tid; j < 4 * 256; j += NT) h[j] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
        const uint32_t k = ks[i];
        atomicAdd(&sm.hist4[0][k & 255u], 1u);
        atomicAdd(&sm.hist4[1][(k >> 8) & 255u], 1u);
        atomicAdd(&sm.hist4[2][(k >> 16) & 255u], 1u);
        atomicAdd(&sm.hist4[3][k >> 24], 1u);
    }
    __syncthreads();
}

// One stable counting pass over the 8-bit digit at `shift`: (ks, vs) ->
// (kd, vd), using the digit histogram sm.hist4[shift / 8].  Returns false
// (and moves nothing) when every key has the same digit.
//
// Each tile is first ranked (per wave, with 64-lane ballots deciding which
// lanes share a digit), then reordered by digit in LDS, and only then written
// out: consecutive threads then write consecutive positions of one digit's
// run instead of scattering single words across memory, which a single
// compute unit could only issue one cache line at a time.
//
// Buffers are plain pointers: they are written and re-read inside this
// kernel, so none of them may be treated as read-only.
__device__ __forceinline__ bool radix_pass(const uint32_t *ks, const uint32_t *vs, uint32_t *kd,
                                           uint32_t *vd, int n, int shift, SortSmem &sm) {
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const uint32_t *hist = sm.hist4[shift >> 3];
    if (wave == 0) {
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const uint32_t s = h0 + h1 + h2 + h3;
        const uint32_t ex = wave_incl_sum(s) - s;
        sm.base[4 * lane] = ex;
        sm.base[4 * lane + 1] = ex + h0;
        sm.base[4 * lane + 2] = ex + h0 + h1;
        sm.base[4 * lane + 3] = ex + h0 + h1 + h2;
        const uint32_t un = (uint32_t)n;
        const uint64_t one = __ballot(h0 == un || h1 == un || h2 == un || h3 == un);
        if (lane == 0) sm.flag = one ? 1u : 0u;
    }
    __syncthreads();
    if (sm.flag) {
        __syncthreads();
        return false;
    }
    for (int t0 = 0; t0 < n; t0 += TILE) {
        const int wbase = t0 + wave * 64 * E;
        uint32_t k[E], v[E], rk[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = wbase + e * 64 + lane;
            k[e] = i < n ? ks[i] : 0u;
            v[e] = i < n ? vs[i] : 0u;
        }
        for (int j = lane; j < 256; j += 64) sm.wcnt[wave][j] = 0;
        // rank of each element among this wave's elements with the same digit
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool valid = wbase + e * 64 + lane < n;
            const uint32_t d = (k[e] >> shift) & 255u;
            uint64_t peers = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const bool bit = (d >> b) & 1u;
                const uint64_t m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            const uint32_t r_in = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(peers >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
            const uint32_t before = sm.wcnt[wave][d];
            rk[e] = before + r_in;
            // the lowest lane of each digit group advances the wave's count;
            // the read above precedes this write in the wave's LDS order
            if (valid && r_in == 0) sm.wcnt[wave][d] = before + (uint32_t)__popcll(peers);
        }
        __syncthreads();
        // per digit: offsets of the waves inside the tile, and the tile count
        if (tid < 256) {
            uint32_t run = 0;
#pragma unroll
            for (int wv = 0; wv < NWAVES; ++wv) {
                const uint32_t c = sm.wcnt[wv][tid];
                sm.wpre[wv][tid] = run;
                run += c;
            }
            sm.tcnt[tid] = run;
        }
        __syncthreads();
        // digit runs inside the staged tile
        if (wave == 0) {
            const uint32_t h0 = sm.tcnt[4 * lane], h1 = sm.tcnt[4 * lane + 1];
            const uint32_t h2 = sm.tcnt[4 * lane + 2], h3 = sm.tcnt[4 * lane + 3];
            const uint32_t s = h0 + h1 + h2 + h3;
            const uint32_t ex = wave_incl_sum(s) - s;
            const uint32_t tb[4] = {ex, ex + h0, ex + h0 + h1, ex + h0 + h1 + h2};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sm.tbase[4 * lane + j] = tb[j];
                sm.gsh[4 * lane + j] = (int32_t)sm.base[4 * lane + j] - (int32_t)tb[j];
            }
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (wbase + e * 64 + lane < n) {
                const uint32_t d = (k[e] >> shift) & 255u;
                const uint32_t slot = sm.tbase[d] + sm.wpre[wave][d] + rk[e];
                sm.stage_k[slot] = k[e];
                sm.stage_v[slot] = v[e];
            }
        }
        __syncthreads();
        const int count = n - t0 < TILE ? n - t0 : TILE;
        for (int s = tid; s < count; s += NT) {
            const uint32_t key = sm.stage_k[s];
            const int pos = s + sm.gsh[(key >> shift) & 255u];
            kd[pos] = key;
            vd[pos] = sm.stage_v[s];
        }
        if (tid < 256) sm.base[tid] += sm.tcnt[tid];
        __syncthreads();
    }
    return true;
}

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

__device__ __forceinline__ uint32_t class_key(const int32_t *cls, uint32_t i) {
    // signed -> unsigned with the same order
    return cls ? ((uint32_t)cls[i] ^ 0x80000000u) : 0u;
}

__global__ __launch_bounds__(NT) void sort_kernel(SortArgs a) {
    __shared__ SortSmem sm;
    const int tid = threadIdx.x;
    const int n = a.n;
    Work w = a.w;
    uint32_t err = 0;

    // score -> ascending key of descending score
    for (int i = tid; i < n; i += NT) {
        const float s = a.scores[i];
        uint32_t u = __float_as_uint(s);
        if (s != s) err |= ERR_NONFINITE;
        if (u == 0x80000000u) u = 0u;
        const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        w.keys0[i] = ~asc;
        w.vals0[i] = (uint32_t)i;
    }
    __syncthreads();

    // Phase 0 sorts by score.  Grouped input adds phase 1 (class id) and
    // phase 2 (image), each a stable sort of the previous phase's order, so
    // the final order is by (image, class, score, index).  One call site for
    // the pass keeps the kernel small.
    uint32_t *ks = w.keys0, *vs = w.vals0, *kd = w.keys1, *vd = w.vals1;
    const int phases = a.grouped ? 3 : 1;
    for (int phase = 0; phase < phases; ++phase) {
        if (phase == 1) {
            // the plain score order is kept for the final compaction
            for (int p = tid; p < n; p += NT) w.score_order[p] = (int32_t)vs[p];
            if (a.offsets) {
                for (int m = tid; m <= a.num_images; m += NT) {
                    const int64_t o = a.offsets[m];
                    bool bad = (m == 0 && o != 0) || (m == a.num_images && o != (int64_t)n);
                    if (m > 0 && o < a.offsets[m - 1]) bad = true;
                    if (bad) err |= ERR_BAD_OFFSETS;
                }
            }
            for (int p = tid; p < n; p += NT) ks[p] = class_key(a.class_ids, vs[p]);
        } else if (phase == 2) {
            for (int p = tid; p < n; p += NT)
                ks[p] = a.offsets ? image_of(a.offsets, a.num_images, vs[p]) : 0u;
        }
        __syncthreads();
        digit_histograms(ks, n, sm);
        for (int shift = 0; shift < 32; shift += 8) {
            if (radix_pass(ks, vs, kd, vd, n, shift, sm)) {
                uint32_t *t0 = ks; ks = kd; kd = t0;
                uint32_t *t1 = vs; vs = vd; vd = t1;
            }
        }
    }

    for (int p = tid; p < a.npad; p += NT) w.order[p] = p < n ? (int32_t)vs[p] : 0;

    const int W = a.words;
    const int S = a.strip;
    uint32_t num_segments = 1;
    if (a.grouped) {
        // ks holds the image of each sorted position; the class is re-read.
        const int chunk = (n + NT - 1) / NT;
        const int lo = tid * chunk < n ? tid * chunk : n;
        const int hi = lo + chunk < n ? lo + chunk : n;
        auto is_start = [&](int p) -> bool {
            if (p == 0) return true;
            return ks[p] != ks[p - 1] ||
                   class_key(a.class_ids, vs[p]) != class_key(a.class_ids, vs[p - 1]);
        };
        uint32_t cnt = 0, first_end = 0xFFFFFFFFu;
        for (int p = lo; p < hi; ++p) {
            if (is_start(p)) ++cnt;
            const bool end = (p == n - 1) || is_start(p + 1);
            if (end && first_end == 0xFFFFFFFFu) first_end = (uint32_t)p;
        }
        uint32_t total = 0;
        uint32_t seg = block_excl_sum(cnt, sm, &total);
        num_segments = total;
        for (int p = lo; p < hi; ++p) {
            if (is_start(p)) ++seg;
            w.seg[p] = seg - 1;
        }
        for (int p = n + tid; p < a.npad; p += NT) w.seg[p] = 0xFFFFFFFFu;
        // band of each row tile: through the tile holding the end of the
        // segment that contains the tile's last row
        uint32_t next_end = block_suffix_min_after(first_end, sm);
        for (int p = hi - 1; p >= lo; --p) {
            const bool end = (p == n - 1) || is_start(p + 1);
            if (end) next_end = (uint32_t)p;
            if ((p & 63) == 63 || p == n - 1) w.tile_cend[p >> 6] = (int32_t)(next_end >> 6) + 1;
        }
    } else {
        for (int r = tid; r < W; r += NT) w.tile_cend[r] = W;
    }
    __syncthreads();

    // mask work items: row tile r covers strips floor(r/S) .. ceil(cend/S)-1
    const int wchunk = (W + NT - 1) / NT;
    const int rlo = tid * wchunk < W ? tid * wchunk : W;
    const int rhi = rlo + wchunk < W ? rlo + wchunk : W;
    uint32_t items = 0, widest = 0;
    for (int r = rlo; r < rhi; ++r) {
        const int cend = w.tile_cend[r];
        const uint32_t it = (uint32_t)((cend + S - 1) / S - r / S);
        items += it;
        widest = it > widest ? it : widest;
    }
    uint32_t total_items = 0;
    uint32_t base = block_excl_sum(items, sm, &total_items);
    for (int r = rlo; r < rhi; ++r) {
        w.item_base[r] = (int32_t)base;
        const int cend = w.tile_cend[r];
        base += (uint32_t)((cend + S - 1) / S - r / S);
    }
    const uint32_t band = block_max(widest, sm);

    // block-wide OR of the error bits
    if (tid == 0) sm.err = 0;
    __syncthreads();
    if (err) atomicOr(&sm.err, err);
    __syncthreads();
    if (tid == 0) {
        w.item_base[W] = (int32_t)total_items;
        Ctrl *c = w.ctrl;
        c->error = sm.err;
        c->flags = FLAG_POSITIVE_AREAS;
        c->count = 0;
        c->num_items = (int32_t)total_items;
        c->band_stride = (int32_t)(band * (uint32_t)S);
        c->num_segments = (int32_t)num_segments;
        c->fused_done = 0u;
    }
}

}  // namespace

hipError_t launch_sort(const Problem &P, const Layout &L, const Work &w, hipStream_t stream) {
    SortArgs a;
    a.scores = P.scores;
    a.class_ids = P.class_ids;
    a.offsets = P.offsets;
    a.n = P.n;
    a.num_images = P.num_images;
    a.grouped = P.grouped ? 1 : 0;
    a.words = (int)L.words;
    a.npad = (int)L.npad;
    a.strip = P.strip;
    a.w = w;
    hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gnms
