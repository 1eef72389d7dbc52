// Sorting one small image by counting ranks, the input checks and the
// per-call initialisation of the workspace: the device code that the
// ranking-sort launch and the one-launch path for small inputs share.
//
// Greedy NMS visits boxes by score, highest first, with equal scores in input
// order ("LeetCUDA 14-nms", algorithm and data flow, step 1: a stable sort).
#pragma once

#include <cmath>

#include "nms_internal.h"

#pragma clang fp contract(off)

namespace gnms {

// Stores of data that workgroups of the same launch read (COHERENT, the
// one-launch path): device-scope stores, which reach the memory all XCDs
// share instead of sitting in this XCD's L2; otherwise plain stores.
template <bool COHERENT, typename T>
__device__ __forceinline__ void store_x(T *p, T v) {
    if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}
template <bool COHERENT>
__device__ __forceinline__ void store_x(float *p, float v) {
    if constexpr (COHERENT)
        __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}
template <bool COHERENT>
__device__ __forceinline__ void store_x(float4 *p, float4 v) {
    if constexpr (COHERENT) {
        uint64_t *q = reinterpret_cast<uint64_t *>(p);
        __hip_atomic_store(q, (uint64_t)__float_as_uint(v.y) << 32 | __float_as_uint(v.x),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 1, (uint64_t)__float_as_uint(v.w) << 32 | __float_as_uint(v.z),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *p = v;
    }
}
template <bool COHERENT>
__device__ __forceinline__ void store_x(uint2 *p, uint2 v) {
    store_x<COHERENT>(reinterpret_cast<uint64_t *>(p), (uint64_t)v.y << 32 | v.x);
}

struct KeysArgs {
    const float4 *boxes;       // one image: for the extent of the boxes (may be null)
    const float *scores;
    const int32_t *class_ids;  // grouped input only (may be null)
    const int64_t *offsets;    // grouped input only (may be null)
    int num_images;
    int n, npad, words, strip, mstride, tiles, grouped;
    Work w;
};

// Mask work items of row tile r when every row covers all column tiles up to
// W: strips floor(r/S) .. ceil(W/S)-1; returns the first item of row tile r.
__device__ __forceinline__ int32_t item_base_full(int r, int W, int S) {
    const int G = (W + S - 1) / S;
    const int g = r / S, u = r % S;
    return (int32_t)(S * (g * G - g * (g - 1) / 2) + u * (G - g));
}

// Per-call initialisation, spread over the threads gid = 0 .. gsz - 1: the
// side arrays the mask kernel only partly writes, the padding rows of the
// sorted arrays, and (one image) the plan of the mask kernel (every row tile
// covers all column tiles).
template <bool GROUPED, bool COHERENT = false>
__device__ __forceinline__ void per_call_init(const KeysArgs &a, int gid, int gsz) {
    const Work &w = a.w;
    for (int r = gid; r <= a.words; r += gsz) {
        if (!GROUPED) store_x<COHERENT>(&w.item_base[r], item_base_full(r, a.words, a.strip));
        if (r < a.words) {
            if (!GROUPED) store_x<COHERENT>(&w.tile_cend[r], (int32_t)a.words);
            store_x<COHERENT>(&w.tcount[r], 0u);
            store_x<COHERENT>(&w.done[r], 0u);
            if (GROUPED) store_x<COHERENT>(&w.kept[r], (uint64_t)0);  // the grouped sweep ORs segments in
        }
    }
    for (int p = gid; p < a.npad; p += gsz) {
#pragma unroll
        for (int j = 0; j <= NEAR_TILES; ++j)
            store_x<COHERENT>(&w.tnear[(size_t)j * a.npad + p], (uint64_t)0);
        if (p >= a.n) {
            store_x<COHERENT>(&w.order[p], (int32_t)0);
            store_x<COHERENT>(&w.sb[p], make_float4(0.f, 0.f, 0.f, 0.f));
            store_x<COHERENT>(&w.area[p], 0.0f);
            if (GROUPED) store_x<COHERENT>(&w.seg[p], 0xFFFFFFFFu);
            else {
                store_x<COHERENT>(&w.scol[p], COARSE_NONE);
                store_x<COHERENT>(&w.srow[p], COARSE_NO_ROW);
            }
        }
    }
}

// Scores read through the constant address space, which lets the compiler
// use scalar loads where the address is the same for every lane.
typedef const __attribute__((address_space(4))) float *const_scores_t;

// One workgroup of THREADS threads checks every score and box of one image
// of n <= THREADS * PER_THREAD boxes, every load of a round in flight
// together, and writes the control block.  The scores must not be NaN; the
// boxes must be finite (else ERR_NONFINITE); a box with x1 < x2, y1 < y2
// and a finite positive area everywhere lets the mask take its fast form
// (FLAG_ORDERED_BOXES).  boxes may be null (the sort-only test export).
template <int THREADS, int PER_THREAD, bool COHERENT = false>
__device__ __forceinline__ void check_image(const KeysArgs &a, const float4 *boxes,
                                            uint32_t *err_sh, uint32_t *unordered_sh) {
    static_assert(PER_THREAD % 4 == 0, "four rounds of loads");
    const int tid = threadIdx.x;
    const int n = a.n;
    if (tid == 0) {
        *err_sh = 0u;
        *unordered_sh = 0u;
    }
    // Loads from clamped indices, with no branch around them, so that a
    // round's loads are all in flight together; entries past n are then
    // ignored.
    uint32_t err = 0;
    bool finite = true, ordered = true;
    constexpr int H = PER_THREAD / 4;  // four rounds keep the registers few
    if (n > 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float sv[H];
            float4 bb[H];
#pragma unroll
            for (int e = 0; e < H; ++e) {
                const int j = min(tid + (h * H + e) * THREADS, n - 1);
                sv[e] = a.scores[j];
                if (boxes != nullptr) bb[e] = boxes[j];
            }
#pragma unroll
            for (int e = 0; e < H; ++e) {
                if (tid + (h * H + e) * THREADS >= n) continue;
                if (sv[e] != sv[e]) err |= ERR_NONFINITE;
                if (boxes == nullptr) continue;
                const float4 b = bb[e];
                finite = finite && isfinite(b.x) && isfinite(b.y) && isfinite(b.z) &&
                         isfinite(b.w);
                const float ar = (b.z - b.x) * (b.w - b.y);
                ordered = ordered && b.x < b.z && b.y < b.w && ar > 0.0f && ar < INFINITY;
            }
        }
    }
    __syncthreads();
    if (!finite) err |= ERR_NONFINITE;
    if (err) atomicOr(err_sh, err);
    if (!ordered) atomicOr(unordered_sh, 1u);
    __syncthreads();
    if (tid == 0) {
        Ctrl *c = a.w.ctrl;
        store_x<COHERENT>(&c->error, *err_sh);
        store_x<COHERENT>(&c->flags, *unordered_sh ? 0u : FLAG_ORDERED_BOXES);
        store_x<COHERENT>(&c->count, (int32_t)0);
        store_x<COHERENT>(&c->num_items, item_base_full(a.words, a.words, a.strip));
        store_x<COHERENT>(&c->band_stride, (int32_t)a.mstride);
        store_x<COHERENT>(&c->num_segments, (int32_t)1);
        store_x<COHERENT>(&c->sweep_done, 0u);
    }
}

// The sorted positions of the 64 boxes of `chunk`, counted by the WAVES waves
// of one workgroup.  The stable order puts box j before box i iff s_j > s_i,
// or s_j == s_i and j < i (float comparisons order scores exactly as the
// radix keys do: -0 equals +0), so box i's sorted position is the number of
// boxes j that satisfy that.  For j in an earlier 64-box chunk than i this is
// s_j >= s_i, in a later chunk s_j > s_i, and in i's own chunk the index
// decides ties.  A NaN score is an error, but the positions must still be a
// permutation (later kernels index with them): NaN counts as -infinity.
// Comparing a raw s_j with the sanitised s_i gives that already, except that
// for a box whose s_i is -infinity (or NaN) every box of an earlier chunk
// precedes it, NaN or not.  The waves split the chunks among them, each
// reading the scores of a chunk with scalar loads (the same values for every
// lane) and comparing them with the lane's own score; wave 0 adds the waves'
// counts and writes the sorted order, boxes and areas.  part: WAVES x 64
// counts in LDS.
template <int WAVES>
__device__ __forceinline__ void rank_chunk(const KeysArgs &a, const float4 *boxes, int chunk,
                                           uint32_t (*part)[64]) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Work &w = a.w;
    const int n = a.n;
    const int chunks = (n + 63) >> 6;
    const int i = 64 * chunk + lane;
    const const_scores_t sc = (const_scores_t)a.scores;
    const float s_raw = i < n ? a.scores[i] : 0.0f;
    const float si = s_raw != s_raw ? -INFINITY : s_raw;
    // the box wave 0 will place, loaded now
    const float4 bi = wave == 0 && boxes != nullptr && i < n ? boxes[i]
                                                             : make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t cnt_early = 0, cnt = 0, early_chunks = 0;
    for (int c = wave; c < chunks; c += WAVES) {
        const const_scores_t sp = sc + 64 * c;
        const int len = min(64, n - 64 * c);
        if (c != chunk && len == 64) {
            if (c < chunk) {
                ++early_chunks;
#pragma unroll
                for (int t = 0; t < 64; ++t) cnt_early += (uint32_t)(sp[t] >= si);
            } else {
#pragma unroll
                for (int t = 0; t < 64; ++t) cnt += (uint32_t)(sp[t] > si);
            }
        } else {
            // this workgroup's own chunk, or the last, partial one (never
            // an earlier one): lane t holds score 64 c + t
            float mine = lane < len ? a.scores[64 * c + lane] : 0.0f;
            if (mine != mine) mine = -INFINITY;
#pragma unroll 1
            for (int t = 0; t < len; ++t) {
                const float sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), t));
                const bool before = c > chunk ? sj > si : (sj > si || (sj == si && t < lane));
                cnt += (uint32_t)before;
            }
        }
    }
    cnt += si == -INFINITY ? 64u * early_chunks : cnt_early;
    part[wave][lane] = cnt;
    __syncthreads();
    if (wave == 0 && i < n) {
        uint32_t r = 0;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) r += part[v][lane];
        w.order[r] = i;
        if (boxes != nullptr) {
            w.sb[r] = bi;
            w.area[r] = (bi.z - bi.x) * (bi.w - bi.y);
        }
    }
}

// rank_chunk with every score first staged in LDS, for the one-launch path,
// whose preparing workgroups each rank one chunk of an image of n <= MAXN
// boxes and sit on its critical path.  One coalesced round of loads, all in
// flight together (rank_staged_load), replaces a chain of scalar loads per
// chunk; every comparison then reads the scores from LDS, four at a time,
// the same address in every lane (a broadcast), the chunk's own included.
// The caller issues no stores before it: a wait for the loads would wait
// for those stores too.  The
// counts are the same as rank_chunk's; the sorted arrays are written with
// device-scope stores.
template <int WAVES, int MAXN>
struct RankStaged {
    static constexpr int T = WAVES * 64;
    static constexpr int PER = (MAXN + T - 1) / T;
    float v[PER];  // scores tid, tid + T, ... (clamped to n - 1)
    float4 bi;     // wave 0: the box of lane's position in the chunk
};

template <int WAVES, int MAXN>
__device__ __forceinline__ void rank_staged_load(const KeysArgs &a, const float4 *boxes,
                                                 int chunk, RankStaged<WAVES, MAXN> &st) {
    using R = RankStaged<WAVES, MAXN>;
    const int tid = threadIdx.x;
    const int n = a.n;
    const int i = 64 * chunk + (tid & 63);
#pragma unroll
    for (int e = 0; e < R::PER; ++e) st.v[e] = a.scores[min(tid + e * R::T, n - 1)];
    st.bi = tid < 64 && boxes != nullptr && i < n ? boxes[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int WAVES, int MAXN>
__device__ __forceinline__ void rank_staged_finish(const KeysArgs &a, const float4 *boxes,
                                                   int chunk, const RankStaged<WAVES, MAXN> &st,
                                                   float *sc, uint32_t (*part)[64]) {
    using R = RankStaged<WAVES, MAXN>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Work &w = a.w;
    const int n = a.n;
    const int chunks = (n + 63) >> 6;
    const int i = 64 * chunk + lane;
#pragma unroll
    for (int e = 0; e < R::PER; ++e)
        if (tid + e * R::T < n) sc[tid + e * R::T] = st.v[e];
    // pad the last chunk to 64 with -infinity: its padding then precedes
    // nothing (s_j > s_i fails, and s_j >= s_i only for s_i = -infinity,
    // whose earlier-chunk rule does not look at the scores)
    if (tid < 64 && chunks * 64 - n > tid) sc[n + tid] = -INFINITY;
    __syncthreads();
    const float s_raw = i < n ? sc[i] : 0.0f;
    const float si = s_raw != s_raw ? -INFINITY : s_raw;
    uint32_t cnt_early = 0, cnt = 0, early_chunks = 0;
    for (int c = wave; c < chunks; c += WAVES) {
        const float4 *s4 = reinterpret_cast<const float4 *>(sc + 64 * c);
        if (c < chunk) {
            ++early_chunks;
            // (groups of four reads: all sixteen in flight would hold 64
            // registers)
#pragma unroll 1
            for (int t0 = 0; t0 < 16; t0 += 4) {
#pragma unroll
                for (int t = t0; t < t0 + 4; ++t) {
                    const float4 q = s4[t];
                    cnt_early += (uint32_t)(q.x >= si) + (uint32_t)(q.y >= si) +
                                 (uint32_t)(q.z >= si) + (uint32_t)(q.w >= si);
                }
            }
        } else if (c > chunk) {
#pragma unroll 1
            for (int t0 = 0; t0 < 16; t0 += 4) {
#pragma unroll
                for (int t = t0; t < t0 + 4; ++t) {
                    const float4 q = s4[t];
                    cnt += (uint32_t)(q.x > si) + (uint32_t)(q.y > si) + (uint32_t)(q.z > si) +
                           (uint32_t)(q.w > si);
                }
            }
        } else {
            // The own chunk: box j = 64 c + t precedes box i = 64 c + lane
            // iff s_j >= s_i for t < lane and s_j > s_i for t > lane, with
            // NaN as -infinity.  Compared raw, a NaN s_j only differs where
            // s_i is -infinity, and then every earlier box precedes anyway.
            // The -infinity padding past n sits at t > lane and never counts.
            const bool ninf = si == -INFINITY;
#pragma unroll 1
            for (int t0 = 0; t0 < 16; t0 += 4) {
#pragma unroll
                for (int t = t0; t < t0 + 4; ++t) {
                    const float4 q = s4[t];
                    const float sj[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        // bitwise, not short-circuit: no branches per lane
                        const int j = 4 * t + u;
                        cnt += ((uint32_t)(j < lane) & ((uint32_t)ninf | (uint32_t)(sj[u] >= si))) |
                               ((uint32_t)(j > lane) & (uint32_t)(sj[u] > si));
                    }
                }
            }
        }
    }
    cnt += si == -INFINITY ? 64u * early_chunks : cnt_early;
    part[wave][lane] = cnt;
    __syncthreads();
    if (wave == 0 && i < n) {
        uint32_t r = 0;
#pragma unroll
        for (int u = 0; u < WAVES; ++u) r += part[u][lane];
        store_x<true>(&w.order[r], (int32_t)i);
        if (boxes != nullptr) {
            store_x<true>(&w.sb[r], st.bi);
            store_x<true>(&w.area[r], (st.bi.z - st.bi.x) * (st.bi.w - st.bi.y));
        }
    }
}

}  // namespace gnms
