// Stages (c) and (d): the greedy sweep over the suppression bitmask, then the
// compaction that maps kept sorted positions back to input indices.
//
// Sweep ("LeetCUDA 14-nms", Phase 2).  The removed bitmap (one bit per sorted
// box, W = ceil(n/64) words) lives in LDS and the boxes are visited in score
// order, 64 at a time (one row tile, "chunk" c):
//   * resolve: lane k holds the diagonal word M[64c + k][c]; the chunk is
//     settled serially in scalar registers.  The lowest not-yet-removed row k
//     whose diagonal word is nonzero is kept and its word ORed into the
//     chunk's removed word; rows whose diagonal word is zero cannot remove
//     anything inside the chunk, so only rows that survive and suppress cost a
//     step.  Every row still clear at the end is kept.  A row's word only has
//     bits above the row, so a later step never changes an earlier decision.
//   * propagate: each kept row ORs its nonzero words for later column tiles
//     into the bitmap.  The mask kernel lists every row's nonzero words (word
//     index, value); the sweep walks those lists instead of the dense rows,
//     which realistic inputs leave almost entirely zero.  A row whose list
//     overflowed is read densely instead.
// The page's sweep takes one workgroup barrier per box.  Here one wave does
// the whole chain with no barrier at all: LDS operations of one wave complete
// in order, so the ORs of chunk c are visible when chunk c + 1 reads its
// removed word.  The diagonal words and row lists of chunk c + 1 do not
// depend on any decision and are loaded while chunk c is resolved.
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
    const uint32_t *rowcnt;
    const uint32_t *lidx;
    const uint64_t *lval;
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

// What the sweep needs of row 64c + lane: its diagonal word and its list.
struct ChunkRows {
    uint64_t diag;
    uint32_t cnt;
    uint32_t idx[ROW_LIST_CAP];
    uint64_t val[ROW_LIST_CAP];
};

// Loads are unconditional (rows past n and chunks past the end re-read the
// last valid row, and their values are never used) so the loop carries no
// branch around them and the wait for them can be placed by hand.
__device__ __forceinline__ void fetch_chunk(const SweepArgs &a, int c, int stride, ChunkRows &r) {
    const int cc = c < a.words ? c : a.words - 1;
    int p = 64 * cc + (int)(threadIdx.x & 63);
    p = p < a.n ? p : a.n - 1;
    const int col0 = (cc / a.strip) * a.strip;
    const int tile = p >> 6;  // == cc
    r.diag = a.mask[(size_t)p * stride + (size_t)(tile - col0)];
    r.cnt = a.rowcnt[p];
    const uint4 *ip = reinterpret_cast<const uint4 *>(a.lidx + (size_t)p * ROW_LIST_CAP);
    const ulonglong2 *vp = reinterpret_cast<const ulonglong2 *>(a.lval + (size_t)p * ROW_LIST_CAP);
#pragma unroll
    for (int j = 0; j < ROW_LIST_CAP / 4; ++j) {
        const uint4 q = ip[j];
        r.idx[4 * j] = q.x;
        r.idx[4 * j + 1] = q.y;
        r.idx[4 * j + 2] = q.z;
        r.idx[4 * j + 3] = q.w;
    }
#pragma unroll
    for (int j = 0; j < ROW_LIST_CAP / 2; ++j) {
        const ulonglong2 q = vp[j];
        r.val[2 * j] = q.x;
        r.val[2 * j + 1] = q.y;
    }
}

// s_waitcnt vmcnt(0): every vector memory load issued so far has returned.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Settle chunk c from `cur` (already loaded) and propagate its kept rows.
__device__ __forceinline__ void sweep_chunk(const SweepArgs &a, int c, int stride,
                                            const ChunkRows &cur, uint64_t *removed) {
    const int lane = threadIdx.x & 63;
    // keep the compiler from moving this chunk's LDS accesses across the
    // previous chunk's (the hardware keeps one wave's LDS operations in order)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const uint64_t valid = rows_valid(c, a.n);
    const uint64_t nz = __ballot(cur.diag != 0ull);
    uint64_t rem = uniform64(removed[c]);
    uint64_t cand = ~rem & nz & valid;
    while (cand) {
        const int k = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cand));
        rem |= read_lane64(cur.diag, k);
        const uint64_t above = k == 63 ? 0ull : (~0ull << (k + 1));
        cand = ~rem & nz & valid & above;
    }
    if (lane == 0) removed[c] = rem;
    const uint64_t kept = ~rem & valid;
    const bool mine = (kept >> lane) & 1ull;
    if (mine && cur.cnt <= (uint32_t)ROW_LIST_CAP) {
#pragma unroll
        for (int j = 0; j < ROW_LIST_CAP; ++j) {
            const uint32_t w = cur.idx[j];
            if ((uint32_t)j < cur.cnt && w > (uint32_t)c) atomicOr(&removed[w], cur.val[j]);
        }
    }
    // Rows with more nonzero words than their list holds: read the dense
    // rows, four rows and two 64-word blocks per row per round, so that eight
    // loads are in flight at once.
    uint64_t over = __ballot(mine && cur.cnt > (uint32_t)ROW_LIST_CAP);
    if (over) {
        const int cend = a.tile_cend[c];
        const int col0 = (c / a.strip) * a.strip;
        while (over) {
            int kr[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                kr[q] = over ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(over)) : -1;
                over &= over - 1ull;
            }
            for (int w0 = c + 1; w0 < cend; w0 += 128) {
                uint64_t v[4][2];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int w = w0 + 64 * j + lane;
                        v[q][j] = (kr[q] >= 0 && w < cend)
                                      ? a.mask[(size_t)(64 * c + kr[q]) * stride + (size_t)(w - col0)]
                                      : 0ull;
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (v[q][j]) atomicOr(&removed[w0 + 64 * j + lane], v[q][j]);
                }
            }
        }
    }
}

__global__ __launch_bounds__(NT) void sweep_kernel(SweepArgs a) {
    extern __shared__ uint64_t removed[];
    __shared__ uint32_t part[NWAVES], part2[NWAVES], tot;
    const int tid = threadIdx.x;
    const int W = a.words, n = a.n;
    const int stride = a.grouped ? a.ctrl->band_stride : a.mstride;

    for (int w = tid; w < W; w += NT) removed[w] = 0ull;
    __syncthreads();

    if ((tid >> 6) == 0) {
        // two register sets, alternating, so the prefetch needs no copies
        // Each step first waits for the rows loaded in the previous step,
        // then issues the loads for the next chunk, then settles this one:
        // the loads of chunk c + 1 fly while chunk c is being resolved.
        ChunkRows ra, rb;
        fetch_chunk(a, 0, stride, ra);
        for (int c = 0; c < W; c += 2) {
            wait_loads();
            fetch_chunk(a, c + 1, stride, rb);
            sweep_chunk(a, c, stride, ra, removed);
            if (c + 1 >= W) break;
            wait_loads();
            fetch_chunk(a, c + 2, stride, ra);
            sweep_chunk(a, c + 1, stride, rb, removed);
        }
    }
    __syncthreads();

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
    a.rowcnt = w.rowcnt;
    a.lidx = w.lidx;
    a.lval = w.lval;
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
