// Stage (a): stable LSD radix sort over all compute units, fused with the
// sorted box gather, and (grouped input) the segment plan of the mask.
//
// Greedy NMS visits boxes by score, highest first, with equal scores in input
// order ("LeetCUDA 14-nms", algorithm and data flow, step 1: a stable sort).
// Each score maps to a 32-bit key whose ascending order is descending score
// (-0.0 folded onto +0.0 so the two tie); stable passes over 8-bit digits
// starting from input order leave equal keys in ascending index order, so
// the index never takes part in a pass.  Grouped input (class ids and/or
// several images) continues with stable passes on the class key and then on
// the image, which makes every (image, class) group contiguous, in score
// order inside; the order after the score passes is kept as the plain score
// order for the final compaction.
//
// Grouped input of up to 131072 boxes, and one image of 16385 to 131072,
// take the same passes in one launch instead (team_sort.hip); the kernels
// below sort the rest, and plan the segments of every grouped input.
//
//   rank_sort_kernel    one image of at most 16384 boxes: every box's sorted
//                       position counted directly (n^2 comparisons), the
//                       sorted-box gather, the input checks and the per-call
//                       initialisation, in one launch.
//   radix_keys_kernel   one workgroup per tile of 2048 boxes: the keys (score;
//                       grouped: class key and image of every box), each
//                       tile's histograms of every digit (digit counts do not
//                       depend on the order, so one read serves all passes),
//                       the input checks and the per-call initialisation.
//   radix_plan_kernel   one workgroup: per pass the global digit counts, their
//                       prefix (where each digit's run starts), whether the
//                       pass can be skipped (every key has the same digit),
//                       which buffer it reads, and which pass is the last.
//   radix_pass_kernel   one workgroup per tile, one launch per pass.  A tile
//                       is ranked (64-lane ballots tell which lanes share a
//                       digit; walking waves, then elements, then lanes walks
//                       indices in order, which keeps the pass stable), its
//                       per-digit offset among earlier tiles comes from a
//                       decoupled look-back over the tiles' published counts,
//                       and the tile is reordered by digit in LDS so that the
//                       writes are coalesced runs.  The last pass writes the
//                       sorted order, the sorted boxes and areas and (grouped)
//                       the inverse permutation.
//   group_starts_kernel grouped input, all compute units: a bitmap of the
//                       sorted positions where a new (image, class) group starts.
//   group_plan_kernel   grouped input, a workgroup per 32 row tiles: segment
//                       of every sorted position, the band of column tiles of
//                       every row tile and the mask work items.
//
// The look-back waits only on lower-numbered tiles, whose workgroups the GPU
// started earlier, and every wait is bounded: a wait that gives up raises an
// internal error instead of hanging.
#include <cmath>

#include "greedy_nms.h"
#include "nms_internal.h"
#include "rank_core.h"
#include "sort_core.h"

#pragma clang fp contract(off)

namespace gnms {
namespace {

using namespace sortcore;

constexpr int NT = RADIX_THREADS;
constexpr int NWAVES = NT / 64;
constexpr int E = RADIX_E;
constexpr int TILE = RADIX_TILE;

constexpr uint32_t LB_AGGREGATE = 1u << 30;  // count of this tile alone
constexpr uint32_t LB_INCLUSIVE = 2u << 30;  // count of this tile and all before it
constexpr uint32_t LB_COUNT = (1u << 30) - 1u;
constexpr uint32_t LB_SPIN_LIMIT = 1u << 22;
constexpr int LB_WINDOW = 16;

// One image needs the score digits only (a third of the LDS to clear).
template <bool GROUPED>
__global__ __launch_bounds__(NT) void radix_keys_kernel(KeysArgs a) {
    constexpr int DIGITS = GROUPED ? RADIX_PASSES : 4;
    __shared__ uint32_t hcopy[HIST_COPIES][DIGITS][256];
    __shared__ uint32_t err_sh;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int tile = blockIdx.x;
    const Work &w = a.w;
    for (int j = tid; j < HIST_COPIES * DIGITS * 256; j += NT) (&hcopy[0][0][0])[j] = 0u;
    if (tid == 0) err_sh = 0u;
    __syncthreads();
    uint32_t (*hist)[256] = hcopy[lane % HIST_COPIES];
    uint32_t err = 0;
    const int base = tile * TILE + wave * 64 * E + lane;
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = base + e * 64;
        s[e] = i < a.n ? a.scores[i] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = base + e * 64;
        if (i < a.n) {
            if (s[e] != s[e]) err |= ERR_NONFINITE;
            const uint32_t k = score_key(s[e]);
            w.keys0[i] = k;
            w.vals0[i] = (uint32_t)i;
            atomicAdd(&hist[0][k & 255u], 1u);
            atomicAdd(&hist[1][(k >> 8) & 255u], 1u);
            atomicAdd(&hist[2][(k >> 16) & 255u], 1u);
            atomicAdd(&hist[3][k >> 24], 1u);
            if constexpr (GROUPED) {
                // the plain score order, should every score pass be skipped
                w.score_order[i] = i;
                const uint32_t c = a.class_ids ? class_key(a.class_ids[i]) : 0u;
                const uint32_t m = a.offsets ? image_of(a.offsets, a.num_images, i) : 0u;
                w.gcls[i] = c;
                w.gimg[i] = m;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    atomicAdd(&hist[4 + d][(c >> (8 * d)) & 255u], 1u);
                    atomicAdd(&hist[8 + d][(m >> (8 * d)) & 255u], 1u);
                }
            }
        }
    }
    if constexpr (!GROUPED) {
        // extent of this tile's boxes (every coordinate), for the quantised
        // overlap pre-test; non-finite values make the pre-test pass
        // everything, and such input is reported as an error anyway
        __shared__ float4 ext_sh[NT / 64];
        float4 ex = make_float4(INFINITY, INFINITY, -INFINITY, -INFINITY);
        if (a.boxes) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int i = base + e * 64;
                if (i < a.n) {
                    const float4 b = a.boxes[i];
                    ex.x = fminf(ex.x, fminf(b.x, b.z));
                    ex.y = fminf(ex.y, fminf(b.y, b.w));
                    ex.z = fmaxf(ex.z, fmaxf(b.x, b.z));
                    ex.w = fmaxf(ex.w, fmaxf(b.y, b.w));
                }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            ex.x = fminf(ex.x, __shfl_xor(ex.x, o, 64));
            ex.y = fminf(ex.y, __shfl_xor(ex.y, o, 64));
            ex.z = fmaxf(ex.z, __shfl_xor(ex.z, o, 64));
            ex.w = fmaxf(ex.w, __shfl_xor(ex.w, o, 64));
        }
        if (lane == 0) ext_sh[wave] = ex;
        __syncthreads();
        if (tid == 0) {
            float4 t = ext_sh[0];
            for (int v = 1; v < NT / 64; ++v) {
                t.x = fminf(t.x, ext_sh[v].x);
                t.y = fminf(t.y, ext_sh[v].y);
                t.z = fmaxf(t.z, ext_sh[v].z);
                t.w = fmaxf(t.w, ext_sh[v].w);
            }
            w.tile_ext[tile] = t;
        }
    }
    const int gid = tile * NT + tid, gsz = a.tiles * NT;
    // batch offsets must rise from 0 to n
    if (GROUPED && a.offsets) {
        for (int m = gid; m <= a.num_images; m += gsz) {
            const int64_t o = a.offsets[m];
            bool bad = (m == 0 && o != 0) || (m == a.num_images && o != (int64_t)a.n);
            if (m > 0 && o < a.offsets[m - 1]) bad = true;
            if (bad) err |= ERR_BAD_OFFSETS;
        }
    }
    if (err) atomicOr(&err_sh, err);
    __syncthreads();
    for (int j = tid; j < DIGITS * 256; j += NT) {
        uint32_t sum = 0;
#pragma unroll
        for (int q = 0; q < HIST_COPIES; ++q) sum += (&hcopy[q][0][0])[j];
        w.hist_tile[(size_t)tile * RADIX_PASSES * 256 + j] = sum;
    }
    // every pass's look-back words of this tile start empty
    for (int j = tid; j < DIGITS * 256; j += NT) {
        const int pass = j >> 8, d = j & 255;
        w.lb_status[((size_t)pass * a.tiles + tile) * 256 + d] = 0u;
    }
    if (tid == 0) w.err_tile[tile] = err_sh;
    if (tile == 0 && tid == 0) {
        Ctrl *c = w.ctrl;
        c->error = 0u;
        c->flags = FLAG_ORDERED_BOXES;
        c->count = 0;
        c->num_items = GROUPED ? 0 : item_base_full(a.words, a.words, a.strip);
        c->band_stride = a.mstride;
        c->num_segments = 1;
        c->sweep_done = 0u;
    }
    per_call_init<GROUPED>(a, gid, gsz);
}

// ---------------------------------------------------------------- rank sort

// One image of at most RANK_SORT_MAX boxes, in one launch: one workgroup per
// 64-box chunk counts the sorted positions of its boxes (n^2 comparisons cost
// less than four passes over few tiles while n is small); an extra
// workgroup checks every score and box and writes the control block beside
// them; every workgroup takes a share of the per-call initialisation.
constexpr int RANK_THREADS = 1024;
constexpr int RANK_WAVES = RANK_THREADS / 64;
constexpr int RANK_PER_THREAD = RANK_SORT_MAX / RANK_THREADS;  // inputs each thread checks
static_assert(RANK_PER_THREAD * RANK_THREADS == RANK_SORT_MAX, "rank sort tiling");

__global__ __launch_bounds__(RANK_THREADS) __attribute__((amdgpu_waves_per_eu(8))) void rank_sort_kernel(
    KeysArgs a, const float4 *boxes) {
    __shared__ uint32_t part[RANK_WAVES][64];
    __shared__ uint32_t err_sh, unordered_sh;
    per_call_init<false>(a, blockIdx.x * RANK_THREADS + threadIdx.x, gridDim.x * RANK_THREADS);
    // workgroup 0 checks the input (the sort-only test export passes no
    // boxes); workgroup 1 + k ranks boxes 64 k .. 64 k + 63
    if (blockIdx.x == 0) check_image<RANK_THREADS, RANK_PER_THREAD>(a, boxes, &err_sh, &unordered_sh);
    else rank_chunk<RANK_WAVES>(a, boxes, blockIdx.x - 1, part);
}

struct PlanArgs {
    int n, tiles, passes;
    Work w;
};

constexpr int PLAN_THREADS = 1024;

// One workgroup: for each pass the global start of each digit's run, and
// whether the pass moves anything.  A pass whose digit is the same for every
// key is skipped; the buffer a pass reads is the one the last moving pass
// before it wrote.  If no pass moves, the last pass still runs (as a copy)
// to write the sorted order and boxes.
__global__ __launch_bounds__(PLAN_THREADS) void radix_plan_kernel(PlanArgs a) {
    __shared__ uint32_t tot[RADIX_PASSES][256];
    __shared__ uint32_t skip[RADIX_PASSES];
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const Work &w = a.w;
    // digit totals over all tiles, (pass, digit) pairs spread over the
    // threads, up to HROUND tiles' counts in flight at a time (each round
    // of dependent loads is a trip to memory)
    constexpr int HROUND = 32;
    for (int j = tid; j < a.passes * 256; j += PLAN_THREADS) {
        uint32_t t = 0;
        for (int t0 = 0; t0 < a.tiles; t0 += HROUND) {
            uint32_t c[HROUND];
#pragma unroll
            for (int q = 0; q < HROUND; ++q)
                c[q] = t0 + q < a.tiles ? w.hist_tile[(size_t)(t0 + q) * RADIX_PASSES * 256 + j]
                                        : 0u;
#pragma unroll
            for (int q = 0; q < HROUND; ++q) t += c[q];
        }
        tot[j >> 8][j & 255] = t;
    }
    __syncthreads();
    // one wave per pass: the digit starts and whether every key shares a digit
    for (int pass = wave; pass < a.passes; pass += PLAN_THREADS / 64) {
        scan256(tot[pass], &w.gbase[pass * 256]);
        const uint32_t un = (uint32_t)a.n;
        const bool one = tot[pass][4 * lane] == un || tot[pass][4 * lane + 1] == un ||
                         tot[pass][4 * lane + 2] == un || tot[pass][4 * lane + 3] == un;
        const uint64_t any = __ballot(one);
        if (lane == 0) skip[pass] = any ? 1u : 0u;
    }
    __syncthreads();
    if (tid == 0) {
        int last = -1, last_score = -1;
        for (int p = 0; p < a.passes; ++p)
            if (!skip[p]) {
                last = p;
                if (p < 4) last_score = p;
            }
        if (last < 0) {
            last = a.passes - 1;
            skip[last] = 0u;
        }
        uint32_t moved = 0;
        for (int p = 0; p < a.passes; ++p) {
            RadixPassPlan pl;
            pl.skip = skip[p];
            pl.src = moved & 1u;
            pl.last = p == last ? 1u : 0u;
            pl.last_score = p == last_score ? 1u : 0u;
            w.pass_plan[p] = pl;
            if (!skip[p]) ++moved;
        }
    }
}

struct PassArgs {
    const float4 *boxes;  // the sorted-box gather of the last pass (may be null)
    int n, tiles, pass, grouped;
    // Grouped input runs a plan kernel first (12 passes, most of which skip).
    // One image runs its four passes unconditionally, each summing the
    // tiles' histograms itself, which saves the plan's launch.
    int planned;
    Work w;
};

struct PassSmem {
    uint32_t gbase[256];   // global start of each digit
    uint32_t tcnt[256];    // digit counts of this tile
    uint32_t tbase[256];   // start of each digit's run inside the staged tile
    int32_t gsh[256];      // global position minus staged slot, per digit
    uint32_t wcnt[NWAVES][256];
    uint32_t wpre[NWAVES][256];
    uint32_t stage_k[TILE];
    uint32_t stage_v[TILE];
    uint32_t err;
    uint32_t unordered;
    float4 ext[NWAVES];
};

// Passes 0-3 sort on the score key (read from the key buffer), 4-7 on the
// class key, 8-11 on the image; the last two read the key of each element's
// input index, so only the values move.
__global__ __launch_bounds__(NT) void radix_pass_kernel(PassArgs a) {
    __shared__ PassSmem sm;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const Work &w = a.w;
    RadixPassPlan pl;
    if (a.planned) {
        pl = w.pass_plan[a.pass];
        if (pl.skip) return;
    } else {
        pl.skip = 0u;
        pl.src = (uint32_t)(a.pass & 1);
        pl.last = a.pass == 3 ? 1u : 0u;
        pl.last_score = 0u;
    }
    const int shift = 8 * (a.pass & 3);
    const int kind = a.pass >> 2;  // 0 score, 1 class, 2 image
    const uint32_t *src_k = pl.src ? w.keys1 : w.keys0;
    const uint32_t *src_v = pl.src ? w.vals1 : w.vals0;
    uint32_t *dst_k = pl.src ? w.keys0 : w.keys1;
    uint32_t *dst_v = pl.src ? w.vals0 : w.vals1;
    // Tile t is workgroup t.  The GPU starts workgroups in order, so a tile
    // only ever waits (in the look-back below) on tiles already running;
    // the wait is bounded in any case.  (Numbering tiles by a ticket taken
    // at the start would put a round trip to memory before every load.)
    const int tile = blockIdx.x;
    if (tid == 0) {
        sm.err = 0u;
        sm.unordered = 0u;
    }
    // the tile's values (and score keys) first: no load here depends on
    // another, so they are all in flight together with the counts below
    const int wbase = tile * TILE + wave * 64 * E;
    uint32_t k[E], v[E], rk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = wbase + e * 64 + lane;
        v[e] = i < a.n ? src_v[i] : 0u;
        k[e] = kind == 0 && i < a.n ? src_k[i] : 0u;
    }
    if (a.planned) {
        sm.gbase[tid] = w.gbase[a.pass * 256 + tid];
    } else {
        // global start of each digit: all tiles' counts of this pass's
        // digit, up to HROUND tiles' loads in flight at a time
        constexpr int HROUND = 32;
        const uint32_t *h = w.hist_tile + (size_t)a.pass * 256 + tid;
        constexpr size_t TS = (size_t)RADIX_PASSES * 256;  // one tile's counts
        uint32_t tot = 0;
        for (int t0 = 0; t0 < a.tiles; t0 += HROUND) {
            uint32_t c[HROUND];
#pragma unroll
            for (int j = 0; j < HROUND; ++j)
                c[j] = t0 + j < a.tiles ? h[(size_t)(t0 + j) * TS] : 0u;
#pragma unroll
            for (int j = 0; j < HROUND; ++j) tot += c[j];
        }
        sm.tcnt[tid] = tot;  // scratch until the scan below
        __syncthreads();
        if (wave == 0) scan256(sm.tcnt, sm.gbase);
    }
    __syncthreads();
    if (tid == 0 && pl.last && w.err_tile[tile]) atomicOr(&w.ctrl->error, w.err_tile[tile]);

    // rank the tile
    if (kind != 0) {
        const uint32_t *gk = kind == 1 ? w.gcls : w.gimg;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = wbase + e * 64 + lane;
            k[e] = i < a.n ? gk[v[e]] : 0u;
        }
    }
    for (int j = lane; j < 256; j += 64) sm.wcnt[wave][j] = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool valid = wbase + e * 64 + lane < a.n;
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
        // the lowest lane of each digit group advances the wave's count; the
        // read above precedes this write in the wave's LDS order
        if (valid && r_in == 0) sm.wcnt[wave][d] = before + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    {
        const int d = tid;
        uint32_t run = 0;
#pragma unroll
        for (int wv = 0; wv < NWAVES; ++wv) {
            const uint32_t c = sm.wcnt[wv][d];
            sm.wpre[wv][d] = run;
            run += c;
        }
        sm.tcnt[d] = run;
        // publish this tile's count, then look back over earlier tiles
        uint32_t *mine = &w.lb_status[((size_t)a.pass * a.tiles + tile) * 256 + d];
        __hip_atomic_store(mine, (tile == 0 ? LB_INCLUSIVE : LB_AGGREGATE) | run,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Look back LB_WINDOW tiles per round trip: the window's status
        // words are loaded together, then summed from the nearest tile back
        // to the first one that already holds an inclusive count.
        uint32_t ex = 0;
        int tp = tile - 1;
        uint32_t spins = 0;
        while (tp >= 0) {
            uint32_t st[LB_WINDOW];
#pragma unroll
            for (int j = 0; j < LB_WINDOW; ++j)
                st[j] = tp - j >= 0
                            ? __hip_atomic_load(
                                  &w.lb_status[((size_t)a.pass * a.tiles + (tp - j)) * 256 + d],
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : LB_INCLUSIVE;
            bool done = false, stalled = false;
            uint32_t add = 0;
            int used = 0;
#pragma unroll
            for (int j = 0; j < LB_WINDOW; ++j) {
                if (done || stalled || tp - j < 0) continue;
                const uint32_t flag = st[j] & ~LB_COUNT;
                if (flag == 0u) {
                    stalled = true;  // not published yet: resume here next round
                    continue;
                }
                add += st[j] & LB_COUNT;
                ++used;
                if (flag == LB_INCLUSIVE) done = true;
            }
            ex += add;
            tp -= used;
            if (done || tp < 0) break;
            if (stalled) {
                if (++spins > LB_SPIN_LIMIT) {
                    atomicOr(&sm.err, ERR_INTERNAL);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (tile > 0)
            __hip_atomic_store(mine, LB_INCLUSIVE | (ex + run), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        sm.gsh[d] = (int32_t)(sm.gbase[d] + ex);  // completed below
    }
    __syncthreads();
    if (wave == 0) scan256(sm.tcnt, sm.tbase);
    __syncthreads();
    sm.gsh[tid] -= (int32_t)sm.tbase[tid];
    // reorder the tile by digit in LDS
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (wbase + e * 64 + lane < a.n) {
            const uint32_t d = (k[e] >> shift) & 255u;
            const uint32_t slot = sm.tbase[d] + sm.wpre[wave][d] + rk[e];
            sm.stage_k[slot] = k[e];
            sm.stage_v[slot] = v[e];
        }
    }
    __syncthreads();
    const int count = a.n - tile * TILE < TILE ? a.n - tile * TILE : TILE;
    bool finite = true, ordered = true;
    // one image: the grid of the quantised pre-test, from every tile's extent
    const bool packs = pl.last && !a.grouped && a.boxes != nullptr;
    PackScale ps{0.f, 0.f, 0.f, 0.f};
    if (packs) {
        float4 ex = make_float4(INFINITY, INFINITY, -INFINITY, -INFINITY);
        for (int t = tid; t < a.tiles; t += NT) {
            const float4 te = w.tile_ext[t];
            ex.x = fminf(ex.x, te.x);
            ex.y = fminf(ex.y, te.y);
            ex.z = fmaxf(ex.z, te.z);
            ex.w = fmaxf(ex.w, te.w);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            ex.x = fminf(ex.x, __shfl_xor(ex.x, o, 64));
            ex.y = fminf(ex.y, __shfl_xor(ex.y, o, 64));
            ex.z = fmaxf(ex.z, __shfl_xor(ex.z, o, 64));
            ex.w = fmaxf(ex.w, __shfl_xor(ex.w, o, 64));
        }
        if (lane == 0) sm.ext[wave] = ex;
        __syncthreads();
        ex = sm.ext[0];
        for (int v = 1; v < NWAVES; ++v) {
            ex.x = fminf(ex.x, sm.ext[v].x);
            ex.y = fminf(ex.y, sm.ext[v].y);
            ex.z = fmaxf(ex.z, sm.ext[v].z);
            ex.w = fmaxf(ex.w, sm.ext[v].w);
        }
        ps.x0 = ex.x;
        ps.y0 = ex.y;
        ps.sx = pack_step(ex.x, ex.z);
        ps.sy = pack_step(ex.y, ex.w);
    }
    if (!pl.last) {
        for (int s = tid; s < count; s += NT) {
            const uint32_t key = sm.stage_k[s];
            const int pos = s + sm.gsh[(key >> shift) & 255u];
            const uint32_t val = sm.stage_v[s];
            if (a.grouped && pl.last_score) w.score_order[pos] = (int32_t)val;
            if (kind == 0) dst_k[pos] = key;
            dst_v[pos] = val;
        }
    } else {
        // The sorted order, and (when boxes are given: the sort-only test
        // export passes none) the sorted boxes with their areas.  The box
        // loads of GB elements are issued before any of their stores, which
        // the compiler may not move across one another.
        constexpr int GB = 8;
        for (int s0 = tid; s0 < count; s0 += NT * GB) {
            int pos[GB];
            uint32_t val[GB];
            float4 b[GB];
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                const int s = s0 + j * NT;
                pos[j] = -1;
                val[j] = 0u;
                if (s < count) {
                    const uint32_t key = sm.stage_k[s];
                    pos[j] = s + sm.gsh[(key >> shift) & 255u];
                    val[j] = sm.stage_v[s];
                }
                b[j] = a.boxes != nullptr && pos[j] >= 0 ? a.boxes[val[j]]
                                                         : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                if (pos[j] < 0) continue;
                if (a.grouped && pl.last_score) w.score_order[pos[j]] = (int32_t)val[j];
                w.order[pos[j]] = (int32_t)val[j];
                if (a.grouped) w.inv[val[j]] = pos[j];
                if (a.boxes == nullptr) continue;
                const float4 bj = b[j];
                finite = finite && isfinite(bj.x) && isfinite(bj.y) && isfinite(bj.z) &&
                         isfinite(bj.w);
                const float ar = (bj.z - bj.x) * (bj.w - bj.y);
                ordered = ordered && bj.x < bj.z && bj.y < bj.w && ar > 0.0f && ar < INFINITY;
                w.sb[pos[j]] = bj;
                w.area[pos[j]] = ar;
                if (packs) {
                    const uint2 crs = coarse_words(bj, ps);
                    w.scol[pos[j]] = crs.x;
                    w.srow[pos[j]] = crs.y;
                }
            }
        }
    }
    if (pl.last) {
        if (!finite) atomicOr(&sm.err, ERR_NONFINITE);
        if (!ordered) atomicOr(&sm.unordered, 1u);
    }
    __syncthreads();
    if (tid == 0) {
        if (sm.err) atomicOr(&w.ctrl->error, sm.err);
        if (sm.unordered) atomicAnd(&w.ctrl->flags, ~FLAG_ORDERED_BOXES);
    }
}

// ---------------------------------------------------------------- grouped plan

constexpr int GP_THREADS = 1024;
constexpr int GP_WAVES = GP_THREADS / 64;
constexpr int GP_TILES = 32;  // row tiles a group-plan workgroup writes

struct GroupPlanArgs {
    int n, words, npad, strip;
    Work w;
};

// Grouped input after the sort, on all compute units: bit p of start_bits
// says a segment (a new (image, class) group) starts at sorted position p.
__global__ __launch_bounds__(256) void group_starts_kernel(GroupPlanArgs a) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    const Work &w = a.w;
    bool st = false;
    if (p < a.n) {
        if (p == 0) {
            st = true;
        } else {
            // clamped: a sort that gave up may leave stale entries (the
            // call's result is then discarded)
            const uint32_t last = (uint32_t)(a.n - 1);
            const uint32_t i = min((uint32_t)w.order[p], last);
            const uint32_t j = min((uint32_t)w.order[p - 1], last);
            st = w.gimg[i] != w.gimg[j] || w.gcls[i] != w.gcls[j];
        }
    }
    const uint64_t m = __ballot(st);
    if ((threadIdx.x & 63) == 0 && p < a.n) w.start_bits[p >> 6] = m;
}

struct GroupPlanSmem {
    uint64_t start[(NMS_MAX_BOXES + 63) / 64];  // bit p: a segment starts at sorted position p
    uint32_t wpre[(NMS_MAX_BOXES + 63) / 64];   // segment starts in the words before
    uint32_t part[GP_WAVES], part2[GP_WAVES], total;
};

// Exclusive workgroup-wide prefix sum; *total receives the sum.
__device__ uint32_t gp_excl_sum(uint32_t v, GroupPlanSmem &sm, uint32_t *total) {
    const int lane = lane_id(), wave = wave_id();
    const uint32_t incl = wave_incl_sum(v);
    if (lane == 63) sm.part[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t s = lane < GP_WAVES ? sm.part[lane] : 0u;
        const uint32_t si = wave_incl_sum(s);
        if (lane < GP_WAVES) sm.part2[lane] = si - s;
        if (lane == GP_WAVES - 1) sm.total = si;
    }
    __syncthreads();
    const uint32_t r = sm.part2[wave] + incl - v;
    *total = sm.total;
    __syncthreads();
    return r;
}

// Position of segment start k (0-based): the word holding it is the last
// word with fewer starts before it than k + 1, then the bit inside it.
__device__ __forceinline__ int start_position(const GroupPlanSmem &sm, int nw, uint32_t k) {
    int lo = 0, hi = nw - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sm.wpre[mid] <= k) lo = mid;
        else hi = mid - 1;
    }
    uint64_t x = sm.start[lo];
    uint32_t j = k - sm.wpre[lo];  // j-th set bit of x (0-based)
    int pos = 0;
#pragma unroll
    for (int width = 32; width > 0; width >>= 1) {
        const uint32_t c = (uint32_t)__popcll(x & ((1ull << width) - 1ull));
        if (j >= c) {
            j -= c;
            x >>= width;
            pos += width;
        }
    }
    return 64 * lo + pos;
}

// One past the last column tile of row tile r's band: its columns run
// through the tile holding the end of the segment that holds the tile's
// last row.
__device__ __forceinline__ int band_end(const GroupPlanSmem &sm, int r, int n, int nw,
                                        uint32_t segments) {
    const int last = 64 * r + 63 < n - 1 ? 64 * r + 63 : n - 1;
    const uint64_t bits = sm.start[last >> 6];
    const uint32_t s =
        sm.wpre[last >> 6] + (uint32_t)__popcll(bits & (~0ull >> (63 - (last & 63)))) - 1u;
    const int end = s + 1u < segments ? start_position(sm, nw, s + 1u) - 1 : n - 1;
    return (end >> 6) + 1;
}

// Grouped input after the sort: segment ids, the band of every row tile and
// its mask work items, the mask row stride.  Workgroup b writes row tiles
// [GP_TILES b, GP_TILES (b + 1)) and their rows; every workgroup derives the
// prefixes it needs (segment starts before each word, work items before
// each tile) from the whole start bitmap itself, which costs O(n / 64).
__global__ __launch_bounds__(GP_THREADS) void group_plan_kernel(GroupPlanArgs a) {
    __shared__ GroupPlanSmem sm;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const Work &w = a.w;
    const int n = a.n, W = a.words, S = a.strip;
    const int nw = (n + 63) / 64;
    const int r0 = (int)blockIdx.x * GP_TILES;
    const int r1 = r0 + GP_TILES < W ? r0 + GP_TILES : W;
    // the segment starts, from group_starts_kernel
    for (int wi = tid; wi < nw; wi += GP_THREADS) sm.start[wi] = w.start_bits[wi];
    __syncthreads();
    // segment starts in the words before each word
    const int chunk = (nw + GP_THREADS - 1) / GP_THREADS;
    const int lo = tid * chunk < nw ? tid * chunk : nw;
    const int hi = lo + chunk < nw ? lo + chunk : nw;
    uint32_t cnt = 0;
    for (int wi = lo; wi < hi; ++wi) cnt += (uint32_t)__popcll(sm.start[wi]);
    uint32_t segments = 0;
    uint32_t before = gp_excl_sum(cnt, sm, &segments);
    for (int wi = lo; wi < hi; ++wi) {
        sm.wpre[wi] = before;
        before += (uint32_t)__popcll(sm.start[wi]);
    }
    __syncthreads();
    // segment id of this workgroup's rows: a wave per word, a lane per row
    for (int wi = r0 + wave; wi < r1; wi += GP_WAVES) {
        const int p = 64 * wi + lane;
        if (p < n) {
            const uint64_t bits = sm.start[wi];
            const uint32_t sg = sm.wpre[wi] + (uint32_t)__popcll(bits & (~0ull >> (63 - lane))) - 1u;
            w.seg[p] = sg;
            if ((bits >> lane) & 1ull) w.seg_start[sg] = p;
        }
    }
    // the band and work items of every row tile (for the prefix), kept for
    // this workgroup's tiles
    const int tchunk = (W + GP_THREADS - 1) / GP_THREADS;
    const int rlo = tid * tchunk < W ? tid * tchunk : W;
    const int rhi = rlo + tchunk < W ? rlo + tchunk : W;
    uint32_t items = 0, widest = 0;
    for (int r = rlo; r < rhi; ++r) {
        const int cend = band_end(sm, r, n, nw, segments);
        const uint32_t it = (uint32_t)((cend + S - 1) / S - r / S);
        items += it;
        widest = it > widest ? it : widest;
    }
    uint32_t total_items = 0;
    uint32_t base = gp_excl_sum(items, sm, &total_items);
    if (rhi > r0 && rlo < r1) {
        for (int r = rlo; r < rhi; ++r) {
            const int cend = band_end(sm, r, n, nw, segments);
            const uint32_t it = (uint32_t)((cend + S - 1) / S - r / S);
            if (r >= r0 && r < r1) {
                w.tile_cend[r] = cend;
                w.item_base[r] = (int32_t)base;
            }
            base += it;
        }
    }
    if (blockIdx.x != 0) return;
    // the widest band sets the row stride of the mask
    uint32_t wmax = widest;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_xor(wmax, o, 64);
        wmax = wmax > u ? wmax : u;
    }
    if (lane == 0) sm.part[wave] = wmax;
    __syncthreads();
    if (tid == 0) {
        uint32_t band = 0;
        for (int i = 0; i < GP_WAVES; ++i) band = sm.part[i] > band ? sm.part[i] : band;
        w.item_base[W] = (int32_t)total_items;
        Ctrl *c = w.ctrl;
        c->num_items = (int32_t)total_items;
        c->band_stride = (int32_t)(band * (uint32_t)S);
        c->num_segments = (int32_t)segments;
        w.seg_start[segments] = n;
    }
}

}  // namespace

// Grouped input, once sorted: the segment starts, then the plan.
static hipError_t launch_group_plan(const Problem &P, const Layout &L, const Work &w,
                                    hipStream_t stream) {
    GroupPlanArgs ga;
    ga.n = P.n;
    ga.words = (int)L.words;
    ga.npad = (int)L.npad;
    ga.strip = P.strip;
    ga.w = w;
    hipLaunchKernelGGL(group_starts_kernel, dim3((unsigned)((P.n + 255) / 256)), dim3(256), 0,
                       stream, ga);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(group_plan_kernel, dim3((unsigned)((L.words + GP_TILES - 1) / GP_TILES)),
                       dim3(GP_THREADS), 0, stream, ga);
    return hipGetLastError();
}

hipError_t launch_radix_sort(const Problem &P, const Layout &L, const Work &w, uint64_t epoch,
                             hipStream_t stream) {
    const int tiles = (int)L.tiles;
    KeysArgs ka;
    ka.boxes = reinterpret_cast<const float4 *>(P.boxes);
    ka.scores = P.scores;
    ka.class_ids = P.class_ids;
    ka.offsets = P.offsets;
    ka.num_images = P.num_images;
    ka.n = P.n;
    ka.npad = (int)L.npad;
    ka.words = (int)L.words;
    ka.strip = P.strip;
    ka.mstride = (int)L.mstride;
    ka.tiles = tiles;
    ka.grouped = P.grouped ? 1 : 0;
    ka.w = w;
    if (!P.grouped && P.n <= RANK_SORT_MAX) {
        const float4 *bx = reinterpret_cast<const float4 *>(P.boxes);
        hipLaunchKernelGGL(rank_sort_kernel, dim3((unsigned)L.words + 1u), dim3(RANK_THREADS), 0,
                           stream, ka, bx);
        return hipGetLastError();
    }
    if (P.sample_sort && P.team_sort && w.team != nullptr && team_sample_applies(P))
        return launch_team_sample(P, L, w, epoch, stream);
    hipError_t e = hipSuccess;
    const bool team = P.team_sort && w.team != nullptr && team_sort_applies(P);
    if (team) {
        e = launch_team_sort(P, L, w, epoch, stream);
        if (e != hipSuccess || !P.grouped) return e;
    } else if (P.grouped) {
        hipLaunchKernelGGL(radix_keys_kernel<true>, dim3(tiles), dim3(NT), 0, stream, ka);
        e = hipGetLastError();
    } else {
        hipLaunchKernelGGL(radix_keys_kernel<false>, dim3(tiles), dim3(NT), 0, stream, ka);
        e = hipGetLastError();
    }
    // The image index of a box is below num_images, so the image digits
    // above those needed for num_images - 1 are 0 for every box: those
    // passes would be skipped anyway and are not launched at all (a skipped
    // pass still costs a launch).  The class key's range is not known here.
    int image_digits = 0;
    for (int64_t m = (int64_t)P.num_images - 1; m > 0; m >>= 8) ++image_digits;
    const int passes = P.grouped ? 8 + image_digits : 4;
    if (e == hipSuccess && P.grouped && !team) {
        PlanArgs pa;
        pa.n = P.n;
        pa.tiles = tiles;
        pa.passes = passes;
        pa.w = w;
        hipLaunchKernelGGL(radix_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, pa);
        e = hipGetLastError();
    }
    for (int pass = 0; pass < passes && e == hipSuccess && !team; ++pass) {
        PassArgs pa;
        pa.boxes = reinterpret_cast<const float4 *>(P.boxes);
        pa.n = P.n;
        pa.tiles = tiles;
        pa.pass = pass;
        pa.grouped = P.grouped ? 1 : 0;
        pa.planned = P.grouped ? 1 : 0;
        pa.w = w;
        hipLaunchKernelGGL(radix_pass_kernel, dim3(tiles), dim3(NT), 0, stream, pa);
        e = hipGetLastError();
    }
    if (e == hipSuccess && P.grouped) e = launch_group_plan(P, L, w, stream);
    return e;
}

}  // namespace gnms
