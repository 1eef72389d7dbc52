// Stage (a) for one image: stable LSD radix sort over all compute units,
// fused with the sorted box gather.
//
// Greedy NMS visits boxes by score, highest first, with equal scores in input
// order ("LeetCUDA 14-nms", algorithm and data flow, step 1: a stable sort).
// Each score maps to a 32-bit key whose ascending order is descending score
// (-0.0 folded onto +0.0 so the two tie); four stable passes over 8-bit digits
// starting from input order leave equal keys in ascending index order, so the
// index never takes part in a pass.
//
//   radix_keys_kernel   one workgroup per tile of 4096 boxes: keys, each
//                       tile's histogram of all four digits (digit counts do
//                       not depend on the order, so one read serves all
//                       passes), and the per-call initialisation of the
//                       plan, the control block and the sweep's side arrays.
//   radix_pass_kernel   one workgroup per tile, four launches.  A tile is
//                       ranked (64-lane ballots tell which lanes share a
//                       digit; walking waves, then elements, then lanes walks
//                       indices in order, which keeps the pass stable), its
//                       per-digit offset among earlier tiles comes from a
//                       decoupled look-back over the tiles' published counts,
//                       and the tile is reordered by digit in LDS so that the
//                       writes are coalesced runs.  The last pass writes the
//                       sorted order and the sorted boxes and areas directly.
//
// The look-back waits only on tiles that took their ticket earlier, which are
// already running, and every wait is bounded: a wait that gives up raises an
// internal error instead of hanging.
#include <cmath>

#include "nms_internal.h"

#pragma clang fp contract(off)

namespace gnms {
namespace {

constexpr int NT = RADIX_THREADS;
constexpr int NWAVES = NT / 64;
constexpr int E = RADIX_E;
constexpr int TILE = RADIX_TILE;

constexpr uint32_t LB_AGGREGATE = 1u << 30;  // count of this tile alone
constexpr uint32_t LB_INCLUSIVE = 2u << 30;  // count of this tile and all before it
constexpr uint32_t LB_COUNT = (1u << 30) - 1u;
constexpr uint32_t LB_SPIN_LIMIT = 1u << 22;
constexpr int LB_WINDOW = 16;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~asc;
}

struct KeysArgs {
    const float *scores;
    int n, npad, words, strip, mstride, tiles;
    Work w;
};

// Mask work items of row tile r when every row covers all column tiles up to
// W: strips floor(r/S) .. ceil(W/S)-1; returns the first item of row tile r.
__device__ __forceinline__ int32_t item_base_full(int r, int W, int S) {
    const int G = (W + S - 1) / S;
    const int g = r / S, u = r % S;
    return (int32_t)(S * (g * G - g * (g - 1) / 2) + u * (G - g));
}

// Lanes add into HIST_COPIES interleaved copies of the histograms: keys of
// real scores share their top digits (the float exponent), and atomics of
// many lanes on one LDS word serialise.
constexpr int HIST_COPIES = 8;

__global__ __launch_bounds__(NT) void radix_keys_kernel(KeysArgs a) {
    __shared__ uint32_t hcopy[HIST_COPIES][4][256];
    __shared__ uint32_t err_sh;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int tile = blockIdx.x;
    const Work &w = a.w;
    for (int j = tid; j < HIST_COPIES * 4 * 256; j += NT) (&hcopy[0][0][0])[j] = 0u;
    if (tid == 0) err_sh = 0u;
    __syncthreads();
    uint32_t (*hist)[256] = hcopy[lane % HIST_COPIES];
    uint32_t err = 0;
    const int base = tile * TILE + wave * 64 * E + lane;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = base + e * 64;
        if (i < a.n) {
            const float s = a.scores[i];
            if (s != s) err |= ERR_NONFINITE;
            const uint32_t k = score_key(s);
            w.keys0[i] = k;
            w.vals0[i] = (uint32_t)i;
            atomicAdd(&hist[0][k & 255u], 1u);
            atomicAdd(&hist[1][(k >> 8) & 255u], 1u);
            atomicAdd(&hist[2][(k >> 16) & 255u], 1u);
            atomicAdd(&hist[3][k >> 24], 1u);
        }
    }
    if (err) atomicOr(&err_sh, err);
    __syncthreads();
    for (int j = tid; j < 4 * 256; j += NT) {
        uint32_t sum = 0;
#pragma unroll
        for (int q = 0; q < HIST_COPIES; ++q) sum += (&hcopy[q][0][0])[j];
        w.hist_tile[(size_t)tile * 1024 + j] = sum;
    }
    // the four passes' look-back words of this tile start empty
    for (int j = tid; j < 4 * 256; j += NT) {
        const int pass = j >> 8, d = j & 255;
        w.lb_status[((size_t)pass * a.tiles + tile) * 256 + d] = 0u;
    }
    if (tid == 0) w.err_tile[tile] = err_sh;
    if (tile == 0 && tid == 0) {
        for (int p = 0; p < 4; ++p) w.tickets[p] = 0u;
        Ctrl *c = w.ctrl;
        c->error = 0u;
        c->flags = FLAG_POSITIVE_AREAS;
        c->count = 0;
        c->num_items = item_base_full(a.words, a.words, a.strip);
        c->band_stride = a.mstride;
        c->num_segments = 1;
        c->fused_done = 0u;
    }
    // Per-call initialisation, spread over the whole grid: the plan of the
    // mask kernel (every row tile covers all column tiles), the padding rows
    // of the sorted arrays, and the sweep's side arrays that the mask kernel
    // only partly writes.
    const int gid = tile * NT + tid, gsz = a.tiles * NT;
    for (int r = gid; r <= a.words; r += gsz) {
        w.item_base[r] = item_base_full(r, a.words, a.strip);
        if (r < a.words) {
            w.tile_cend[r] = a.words;
            w.tcount[r] = 0u;
            w.done[r] = 0u;
        }
    }
    for (int p = gid; p < a.npad; p += gsz) {
#pragma unroll
        for (int j = 0; j <= NEAR_TILES; ++j) w.tnear[(size_t)j * a.npad + p] = 0ull;
        if (p >= a.n) {
            w.order[p] = 0;
            w.sb[p] = make_float4(0.f, 0.f, 0.f, 0.f);
            w.area[p] = 0.0f;
        }
    }
}

struct PassArgs {
    const uint32_t *src_k, *src_v;
    uint32_t *dst_k, *dst_v;
    const float4 *boxes;  // last pass only: gather the sorted boxes (may be null)
    int n, tiles, pass;
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
    uint32_t part[NWAVES];
    uint32_t tile;
    uint32_t err;
    uint32_t bad_area;
};

// Exclusive scan of v[0..256) into out[] by the first wave (4 per lane).
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

template <bool LAST>
__global__ __launch_bounds__(NT) void radix_pass_kernel(PassArgs a) {
    __shared__ PassSmem sm;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int shift = 8 * a.pass;
    const Work &w = a.w;
    if (tid == 0) {
        // tiles are numbered in the order their workgroups start, so a tile
        // only ever waits on tiles that are already running
        sm.tile = atomicAdd(&w.tickets[a.pass], 1u);
        sm.err = 0u;
        sm.bad_area = 0u;
    }
    __syncthreads();
    const int tile = (int)sm.tile;
    if (a.pass == 0 && tid == 0 && w.err_tile[tile]) atomicOr(&w.ctrl->error, w.err_tile[tile]);

    // global start of each digit: all tiles' counts of this pass's digit
    {
        uint32_t tot = 0;
        for (int t = 0; t < a.tiles; ++t)
            tot += w.hist_tile[(size_t)t * 1024 + a.pass * 256 + tid];
        sm.tcnt[tid] = tot;  // scratch until the scan below
    }
    __syncthreads();
    if (wave == 0) scan256(sm.tcnt, sm.gbase);

    // load and rank the tile
    const int wbase = tile * TILE + wave * 64 * E;
    uint32_t k[E], v[E], rk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = wbase + e * 64 + lane;
        k[e] = i < a.n ? a.src_k[i] : 0u;
        v[e] = i < a.n ? a.src_v[i] : 0u;
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
    bool finite = true, positive = true;
    for (int s = tid; s < count; s += NT) {
        const uint32_t key = sm.stage_k[s];
        const int pos = s + sm.gsh[(key >> shift) & 255u];
        const uint32_t val = sm.stage_v[s];
        if (!LAST) {
            a.dst_k[pos] = key;
            a.dst_v[pos] = val;
        } else {
            // the sorted order, and (when boxes are given: the sort-only test
            // export passes none) the sorted boxes with their areas
            w.order[pos] = (int32_t)val;
            if (a.boxes == nullptr) continue;
            const float4 b = a.boxes[val];
            finite = finite && isfinite(b.x) && isfinite(b.y) && isfinite(b.z) && isfinite(b.w);
            const float ar = (b.z - b.x) * (b.w - b.y);
            positive = positive && ar > 0.0f && ar < INFINITY;
            w.sb[pos] = b;
            w.area[pos] = ar;
        }
    }
    if (LAST) {
        if (!finite) atomicOr(&sm.err, ERR_NONFINITE);
        if (!positive) atomicOr(&sm.bad_area, 1u);
    }
    __syncthreads();
    if (tid == 0) {
        if (sm.err) atomicOr(&w.ctrl->error, sm.err);
        if (sm.bad_area) atomicAnd(&w.ctrl->flags, ~FLAG_POSITIVE_AREAS);
    }
}

}  // namespace

hipError_t launch_radix_sort(const Problem &P, const Layout &L, const Work &w,
                             hipStream_t stream) {
    const int tiles = (int)L.tiles;
    KeysArgs ka;
    ka.scores = P.scores;
    ka.n = P.n;
    ka.npad = (int)L.npad;
    ka.words = (int)L.words;
    ka.strip = P.strip;
    ka.mstride = (int)L.mstride;
    ka.tiles = tiles;
    ka.w = w;
    hipLaunchKernelGGL(radix_keys_kernel, dim3(tiles), dim3(NT), 0, stream, ka);
    hipError_t e = hipGetLastError();
    uint32_t *bk[2] = {w.keys0, w.keys1};
    uint32_t *bv[2] = {w.vals0, w.vals1};
    for (int pass = 0; pass < 4 && e == hipSuccess; ++pass) {
        PassArgs pa;
        pa.src_k = bk[pass & 1];
        pa.src_v = bv[pass & 1];
        pa.dst_k = bk[(pass + 1) & 1];
        pa.dst_v = bv[(pass + 1) & 1];
        pa.boxes = reinterpret_cast<const float4 *>(P.boxes);
        pa.n = P.n;
        pa.tiles = tiles;
        pa.pass = pass;
        pa.w = w;
        if (pass < 3)
            hipLaunchKernelGGL(radix_pass_kernel<false>, dim3(tiles), dim3(NT), 0, stream, pa);
        else
            hipLaunchKernelGGL(radix_pass_kernel<true>, dim3(tiles), dim3(NT), 0, stream, pa);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gnms
