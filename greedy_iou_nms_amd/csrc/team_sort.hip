// Stage (a) in one launch: the stable LSD radix sort of radix.hip (same
// keys, same 8-bit digit passes, same order of passes), run by a team of
// workgroups that stay resident through every pass.  Each pass is one
// round of the team instead of one kernel launch.
//
// Greedy NMS visits boxes by score, highest first, with equal scores in
// input order ("LeetCUDA 14-nms", algorithm and data flow, step 1: a stable
// sort).  Grouped input continues with stable passes on the class key and
// then on the image ("YOLOv5 post-processing", section 2.2: boxes of
// different classes never suppress one another).
//
// Why one launch: at 65,536 boxes a pass moves 0.5 MB, a few hundred
// nanoseconds of HBM time, yet a pass launched as its own kernel took about
// 13 us on this GPU, spent in dependent trips to memory (the tile's loads,
// the look-back, the scatter) and in the kernel's start and end.  Here the
// passes follow one another inside the launch, with no barrier between them.
//
// The team is blocks 0 .. T - 1 (T <= 32, one tile of E * 1024 boxes each),
// which the GPU spreads over its XCDs; the blocks after them ("checkers")
// do the work no pass waits for.  Every word one workgroup hands to another
// goes through device-coherent (agent-scope) loads and stores, whose
// bandwidth is per XCD: a team packed onto one XCD ran its exchanges at a
// fraction of the speed.
//
//   phase 0   member t keys the input tile t (score key; grouped: class key
//             and image), checks its boxes, counts the digits of every pass
//             in LDS and publishes the counts and (one image) its boxes'
//             extent.  Owners then sum groups of 8 columns over all tiles
//             (each digit's total, and every tile's count of it in the tiles
//             before), and every member reads the totals and its own
//             prefixes back.  From the totals every member derives the same
//             plan: a pass whose digit is the same for every key is skipped;
//             the last pass that runs writes the outputs.
//   passes    the first pass sorts the input tiles, whose digit offsets
//             phase 0 gave.  Each later pass loads its tile from a ring of
//             three buffers of tagged words (value, then the pass's key),
//             waiting only for the words it reads; ranks it (64-lane
//             ballots; waves, then elements, then lanes walk positions in
//             order, which keeps the pass stable); publishes the tile's digit
//             counts and sums those of the tiles before it; and writes the
//             tile out in digit runs through LDS, each word tagged with the
//             next pass's tag.  A ring buffer is rewritten only after every
//             member has loaded the pass that last read it (its counts for
//             that pass are out).
//   last pass the sorted order, and (boxes given) the sorted boxes, areas
//             and (one image) the quantised pre-test words; grouped input
//             also the inverse permutation, and the score order after the
//             last score pass.
//   checkers  per-call initialisation for the later kernels and the check of
//             the batch offsets.
//
// Every word one workgroup reads from another carries a tag from the call's
// epoch (and, in the ring, the pass), so nothing an earlier call or pass
// left passes for the one expected; every wait is bounded and a wait that
// gives up raises ERR_INTERNAL.  Member 0 writes the control block last,
// from what every workgroup reported.
#include <cmath>

#include "greedy_nms.h"
#include "nms_internal.h"
#include "rank_core.h"
#include "sort_core.h"

#pragma clang fp contract(off)

namespace gnms {
namespace {

using namespace sortcore;

constexpr int NT = TEAM_THREADS;
constexpr int NW = NT / 64;
constexpr uint32_t TEAM_SPIN_LIMIT = 1u << 18;
constexpr int SLOT = 16;  // words between two workgroups' slots (128 bytes)

// Device-coherent loads and stores (agent scope) for the words workgroups
// hand to one another.
template <typename T>
__device__ __forceinline__ T ld_c(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_c(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): every vector memory access of this wave so far has
// completed (stores included: they have reached the memory all XCDs share).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t v) {
    return (uint64_t)tag << 32 | v;
}

// Loads the tagged words a[m * stride] (and b[m * stride] when b is given),
// for bit m of want, until each carries tag; their values land in va[m]
// (vb[m]).  False when the wait gave up.  Addresses come from one base and a
// stride, which keeps the registers few.
template <int K>
__device__ __forceinline__ bool poll_words(const uint64_t *a, const uint64_t *b, size_t stride,
                                           uint32_t want, uint32_t tag, uint32_t (&va)[K],
                                           uint32_t (&vb)[K]) {
    uint32_t spins = 0;
    while (want) {
        uint64_t wa[K], wb[K];
#pragma unroll
        for (int m = 0; m < K; ++m) {
            const bool on = (want >> m) & 1u;
            wa[m] = on ? ld_c(a + m * stride) : 0ull;
            wb[m] = on && b != nullptr ? ld_c(b + m * stride) : ((uint64_t)tag << 32);
        }
#pragma unroll
        for (int m = 0; m < K; ++m)
            if (((want >> m) & 1u) && (uint32_t)(wa[m] >> 32) == tag &&
                (uint32_t)(wb[m] >> 32) == tag) {
                va[m] = (uint32_t)wa[m];
                vb[m] = (uint32_t)wb[m];
                want &= ~(1u << m);
            }
        if (!want) break;
        if (++spins > TEAM_SPIN_LIMIT) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}

template <int K>
__device__ __forceinline__ bool poll_words(const uint64_t *a, size_t stride, uint32_t want,
                                           uint32_t tag, uint32_t (&va)[K]) {
    uint32_t vb[K];
    return poll_words<K>(a, nullptr, stride, want, tag, va, vb);
}

// The team's words in the workspace (Layout::off_team), for tl members at
// most (the layout's team_layout_members).
struct TeamWork {
    int tl;
    uint64_t *hist;  // [tl][RADIX_PASSES * 256]: member t's digit counts of its input tile
    uint64_t *pre;   // [tl][RADIX_PASSES * 256]: counts in the input tiles before t
    uint64_t *tot;   // [RADIX_PASSES * 256]: digit totals
    uint64_t *cnt;   // [RADIX_PASSES][tl][256]: per pass, tile counts (look-back)
    uint64_t *done;  // [tl][SLOT]: member t finished, with its error bits
    uint64_t *ext;   // [tl][SLOT]: extent of member t's input boxes (words 0-3)
    uint64_t *chk;   // [tl * TEAM_CHECKERS_PER_MEMBER][SLOT]: checker h finished: error bits
    uint64_t *end;   // one past the last word
};

__host__ __device__ inline TeamWork team_work(uint64_t *base, int tl) {
    TeamWork tw;
    uint64_t *p = base;
    tw.tl = tl;
    tw.hist = p;
    p += (size_t)tl * RADIX_PASSES * 256;
    tw.pre = p;
    p += (size_t)tl * RADIX_PASSES * 256;
    tw.tot = p;
    p += (size_t)RADIX_PASSES * 256;
    tw.cnt = p;
    p += (size_t)RADIX_PASSES * tl * 256;
    tw.done = p;
    p += (size_t)tl * SLOT;
    tw.ext = p;
    p += (size_t)tl * SLOT;
    tw.chk = p;
    p += (size_t)tl * TEAM_CHECKERS_PER_MEMBER * SLOT;
    tw.end = p;
    return tw;
}

struct TeamArgs {
    KeysArgs ka;
    int team;      // members (tiles of E * NT input boxes)
    int checkers;  // blocks T .. T + checkers - 1 (0: the members do their work)
    int passes;    // 4, or 8 + the image digits (grouped)
    uint64_t epoch;
    uint64_t *team_ws;
    int tl;        // members the workspace provides for
    // [3][2 * npad] words: the element at position i of a pass's input is
    // (value) at 2 i and (key) at 2 i + 1, each with the pass's ring tag;
    // pass j reads ring j % 3
    uint64_t *ring;
};

// Grouped input of up to TEAM_LDS_OFFSETS - 1 images finds a box's image in
// a copy of the batch offsets in LDS.
constexpr int TEAM_LDS_OFFSETS = 2048;
// Grouped input whose images all hold at most IMAGE_CAP boxes has each
// image's group order sorted in LDS by one checker block (see image_sort).
constexpr int IMAGE_CAP = 4096;

__device__ __forceinline__ uint32_t image_in(const int32_t *off, int num_images, int64_t i) {
    int lo = 0, hi = num_images - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    return (uint32_t)lo;
}

// Tag of the ring words that pass number j (0, 1, ... among the passes that
// run) reads: unique per call and pass.
__device__ __forceinline__ uint32_t ring_tag(uint64_t epoch, int j) {
    return (uint32_t)(epoch * 16u + (uint64_t)j);
}

// Checker error word: bit 31 = some box is not ordered.
constexpr uint32_t UNORDERED_BIT = 0x80000000u;

template <int E, bool GROUPED>
struct TeamSmem {
    static constexpr int S = E * NT;
    static constexpr int DIGITS = GROUPED ? RADIX_PASSES : 4;
    static constexpr int ICAP = GROUPED ? IMAGE_CAP : 1;
    union {
        uint32_t hc[HIST_COPIES][DIGITS][256];
        struct {
            uint32_t k[S];
            uint32_t v[S];
        } stage;
        struct {  // one image's keys and its order, local indices
            uint32_t skey[ICAP];
            uint32_t ckey[ICAP];
            uint32_t perm[2][ICAP];
        } img;
    } u;
    uint32_t gtot[DIGITS * 256];  // digit totals per pass
    uint32_t gpre[DIGITS * 256];  // this tile's input-order prefixes per pass
    uint32_t wcnt[NW][256];
    uint32_t wpre[NW][256];
    uint32_t gb[256];     // start of each digit in the pass's output
    uint32_t tcnt[256];   // digit counts of this tile
    uint32_t tbase[256];  // start of each digit's run in the staged tile
    int32_t gsh[256];     // output position minus staged slot, per digit
    uint32_t part[4][256];
    float4 ext[NW];
    PackScale ps;
    uint32_t skip[RADIX_PASSES];
    int32_t act[RADIX_PASSES];  // the passes that run, in order
    int32_t nact;
    uint32_t err, unordered;
    uint32_t img_bad, img_max;
    // grouped input: the batch offsets (up to TEAM_LDS_OFFSETS - 1 images)
    int32_t offs[GROUPED ? TEAM_LDS_OFFSETS : 1];
};

// ------------------------------------------------------------------ checkers

// Work no pass waits for, spread over H blocks (h = 0 .. H - 1): a share of
// the per-call initialisation for the later kernels, and the check of the
// batch offsets.  Returns this thread's error bits.
template <bool GROUPED>
__device__ uint32_t team_check(const TeamArgs &a, int h, int H) {
    const KeysArgs &ka = a.ka;
    const int gid = h * NT + threadIdx.x, gsz = H * NT;
    per_call_init<GROUPED>(ka, gid, gsz);
    uint32_t err = 0;
    if (GROUPED && ka.offsets) {
        // batch offsets must rise from 0 to n
        for (int m = gid; m <= ka.num_images; m += gsz) {
            const int64_t o = ka.offsets[m];
            bool bad = (m == 0 && o != 0) || (m == ka.num_images && o != (int64_t)ka.n);
            if (m > 0 && o < ka.offsets[m - 1]) bad = true;
            if (bad) err |= ERR_BAD_OFFSETS;
        }
    }
    return err;
}

__device__ __forceinline__ float4 ext_min_max(float4 a, float4 b) {
    return make_float4(fminf(a.x, b.x), fminf(a.y, b.y), fmaxf(a.z, b.z), fmaxf(a.w, b.w));
}

__device__ __forceinline__ float4 wave_ext(float4 ex) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        ex = ext_min_max(ex, make_float4(__shfl_xor(ex.x, o, 64), __shfl_xor(ex.y, o, 64),
                                         __shfl_xor(ex.z, o, 64), __shfl_xor(ex.w, o, 64)));
    return ex;
}

// ------------------------------------------------------------------ images

// Grouped input: copies the batch offsets to LDS (no offsets: one image of
// n boxes) when there are fewer than TEAM_LDS_OFFSETS images, and returns
// whether every image may be sorted in LDS by itself: the offsets rise from
// 0 to n and no image holds more than IMAGE_CAP boxes.  Every block of the
// launch computes the same answer from the same offsets.
template <class Smem>
__device__ bool stage_offsets(const KeysArgs &ka, Smem &sm) {
    const int tid = threadIdx.x;
    const int images = ka.offsets ? ka.num_images : 1;
    if (images >= TEAM_LDS_OFFSETS) return false;
    if (tid == 0) {
        sm.img_bad = 0u;
        sm.img_max = 0u;
    }
    for (int j = tid; j <= images; j += NT)
        sm.offs[j] = ka.offsets ? (int32_t)ka.offsets[j] : (j == 0 ? 0 : ka.n);
    __syncthreads();
    uint32_t bad = 0u, big = 0u;
    for (int m = tid; m < images; m += NT) {
        const int64_t lo = sm.offs[m], hi = sm.offs[m + 1];
        if (hi < lo) bad = 1u;
        else big = (uint32_t)(hi - lo) > big ? (uint32_t)(hi - lo) : big;
    }
    if (sm.offs[0] != 0 || sm.offs[images] != ka.n) bad = 1u;
    if (bad) atomicOr(&sm.img_bad, 1u);
    if (big) atomicMax(&sm.img_max, big);
    __syncthreads();
    return sm.img_bad == 0u && sm.img_max <= (uint32_t)IMAGE_CAP;
}

// Ranks E positions per thread (position wave * 64 E + 64 e + lane, of the
// first `count`) by digit d[e]: rk[e] = positions before it in the same
// wave with the same digit; sm.wcnt[wave][digit] = the wave's count.  The
// lanes with the same digit come from one ballot per bit (a lane keeps the
// lanes whose bit equals its own).
template <int E, class Smem>
__device__ __forceinline__ void rank_digits(Smem &sm, const uint32_t (&d)[E], int count,
                                            uint32_t (&rk)[E]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int q = lane; q < 256; q += 64) sm.wcnt[wave][q] = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool valid = wave * 64 * E + e * 64 + lane < count;
        const uint32_t nd = ~d[e];
        const uint64_t vm = __ballot(valid);
        if (vm == 0ull) {  // no element here: nothing to rank or count
            rk[e] = 0u;
            continue;
        }
        uint32_t plo = (uint32_t)vm, phi = (uint32_t)(vm >> 32);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            // 0 where this lane's bit is set, all ones where it is clear
            const uint32_t tm = (uint32_t)__builtin_amdgcn_sbfe((int)nd, bit, 1);
            const uint64_t m = __ballot(tm == 0u);
            plo &= (uint32_t)m ^ tm;
            phi &= (uint32_t)(m >> 32) ^ tm;
        }
        const uint32_t r_in = __builtin_amdgcn_mbcnt_hi(phi, __builtin_amdgcn_mbcnt_lo(plo, 0u));
        const uint32_t before = sm.wcnt[wave][d[e]];
        rk[e] = before + r_in;
        // the lowest lane of each digit group advances the wave's count; the
        // read above precedes this write in the wave's LDS order
        if (valid && r_in == 0)
            sm.wcnt[wave][d[e]] = before + (uint32_t)(__popc(plo) + __popc(phi));
    }
}

// Slots of one LDS pass, by one wave: sm.wpre[wv][d] = the elements of
// digits below d plus those of digit d in the waves before wv, for the
// first nwa waves (those holding elements; the others counted nothing).
template <class Smem>
__device__ __forceinline__ void digit_slots(Smem &sm, int nwa) {
    const int lane = threadIdx.x & 63;
    uint4 tot = make_uint4(0u, 0u, 0u, 0u);
    for (int wv = 0; wv < nwa; ++wv) {
        const uint4 c = *reinterpret_cast<const uint4 *>(&sm.wcnt[wv][4 * lane]);
        tot.x += c.x;
        tot.y += c.y;
        tot.z += c.z;
        tot.w += c.w;
    }
    const uint32_t sum = tot.x + tot.y + tot.z + tot.w;
    const uint32_t ex = wave_incl_sum(sum) - sum;
    uint4 run = make_uint4(ex, ex + tot.x, ex + tot.x + tot.y, ex + tot.x + tot.y + tot.z);
    for (int wv = 0; wv < nwa; ++wv) {
        const uint4 c = *reinterpret_cast<const uint4 *>(&sm.wcnt[wv][4 * lane]);
        *reinterpret_cast<uint4 *>(&sm.wpre[wv][4 * lane]) = run;
        run.x += c.x;
        run.y += c.y;
        run.z += c.z;
        run.w += c.w;
    }
}

// One image m of at most IMAGE_CAP boxes, by one block: its boxes in group
// order (class key, then score key, then input index: stable 8-bit passes
// in LDS from input order, score digits first) at the image's own
// positions [off[m], off[m + 1]), with the inverse permutation and the
// sorted boxes and areas.  Digits every box of the image shares are
// skipped.
template <class Smem>
__device__ void image_sort(const KeysArgs &ka, Smem &sm, int m) {
    constexpr int EI = IMAGE_CAP / NT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Work &w = ka.w;
    const int base = sm.offs[m], cnt = sm.offs[m + 1] - base;
    if (cnt <= 0) return;
    auto &img = sm.u.img;
    for (int j = tid; j < 8 * 256; j += NT) sm.gtot[j] = 0u;
    __syncthreads();
    // keys, and the digit counts of the eight digits (a digit every lane of
    // a wave shares is one add)
#pragma unroll
    for (int e = 0; e < EI; ++e) {
        const int v = e * NT + tid;
        const bool valid = v < cnt;
        const uint32_t sk = valid ? score_key(ka.scores[base + v]) : 0u;
        const uint32_t ck = valid && ka.class_ids ? class_key(ka.class_ids[base + v]) : 0u;
        if (valid) {
            img.skey[v] = sk;
            img.ckey[v] = ck;
            img.perm[0][v] = (uint32_t)v;
        }
        const uint64_t vm = __ballot(valid);
        if (vm == 0ull) continue;
        const int first = __builtin_ctzll(vm);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t dg = ((q < 4 ? sk : ck) >> (8 * (q & 3))) & 255u;
            const uint32_t d0 = (uint32_t)__shfl((int)dg, first, 64);
            if (__ballot(valid && dg != d0) == 0ull) {
                if (lane == first) atomicAdd(&sm.gtot[q * 256 + d0], (uint32_t)__popcll(vm));
            } else if (valid) {
                atomicAdd(&sm.gtot[q * 256 + dg], 1u);
            }
        }
    }
    __syncthreads();
    if (wave < 8) {
        const uint32_t *g = &sm.gtot[wave * 256];
        const uint32_t un = (uint32_t)cnt;
        const bool one = g[4 * lane] == un || g[4 * lane + 1] == un || g[4 * lane + 2] == un ||
                         g[4 * lane + 3] == un;
        const uint64_t any = __ballot(one);
        if (lane == 0) sm.skip[wave] = any ? 1u : 0u;
    }
    __syncthreads();
    const int nwa = min(NW, (cnt + 64 * EI - 1) / (64 * EI));  // waves holding positions
    int cur = 0;
    for (int q = 0; q < 8; ++q) {
        if (sm.skip[q]) continue;
        const int shift = 8 * (q & 3);
        uint32_t v[EI], d[EI], rk[EI];
#pragma unroll
        for (int e = 0; e < EI; ++e) {
            const int i = wave * 64 * EI + e * 64 + lane;
            v[e] = i < cnt ? img.perm[cur][i] : 0u;
            d[e] = i < cnt ? ((q < 4 ? img.skey[v[e]] : img.ckey[v[e]]) >> shift) & 255u : 0u;
        }
        rank_digits<EI>(sm, d, cnt, rk);
        __syncthreads();
        if (wave == 0) digit_slots(sm, nwa);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EI; ++e)
            if (wave * 64 * EI + e * 64 + lane < cnt)
                img.perm[cur ^ 1][sm.wpre[wave][d[e]] + rk[e]] = v[e];
        __syncthreads();
        cur ^= 1;
    }
    for (int r = tid; r < cnt; r += NT) {
        const int pos = base + r;
        const int i = base + (int)img.perm[cur][r];
        w.order[pos] = i;
        w.inv[i] = pos;
        if (ka.boxes != nullptr) {
            const float4 bj = ka.boxes[i];
            w.sb[pos] = bj;
            w.area[pos] = (bj.z - bj.x) * (bj.w - bj.y);
        }
    }
    __syncthreads();  // the next image reuses the LDS
}

// ------------------------------------------------------------------ kernel

template <int E, bool GROUPED>
__global__ __launch_bounds__(NT) void team_sort_kernel(TeamArgs a) {
    using Smem = TeamSmem<E, GROUPED>;
    constexpr int S = Smem::S;
    __shared__ Smem sm;
    const KeysArgs &ka = a.ka;
    const Work &w = ka.w;
    const TeamWork tw = team_work(a.team_ws, a.tl);
    const uint32_t tag = (uint32_t)a.epoch;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int T = a.team, n = ka.n;
    if (b >= T) {
        // a checker: its error bits, once its work is done
        if (tid == 0) sm.err = 0u;
        __syncthreads();
        const uint32_t e = team_check<GROUPED>(a, b - T, a.checkers);
        if (e) atomicOr(&sm.err, e);
        if constexpr (GROUPED) {
            // every image small enough: this block's share of the images
            if (stage_offsets(ka, sm)) {
                const int images = ka.offsets ? ka.num_images : 1;
                for (int m = b - T; m < images; m += a.checkers) image_sort(ka, sm, m);
            }
        }
        __syncthreads();
        if (tid == 0) st_c(&tw.chk[(size_t)(b - T) * SLOT], tagged(tag, sm.err));
        return;
    }
    // Members are blocks 0 .. T - 1, which the GPU spreads over its XCDs:
    // the passes move data through device-coherent loads and stores, whose
    // bandwidth is per XCD.
    const int t = b;

    // ---------------------------------------------------------- phase 0
    if (tid == 0) {
        sm.err = 0u;
        sm.unordered = 0u;
    }
    __syncthreads();
    if (a.checkers == 0) {
        const uint32_t e = team_check<GROUPED>(a, t, T);
        if (e) atomicOr(&sm.err, e);
    }
    const bool lds_offs = GROUPED && ka.offsets != nullptr && ka.num_images < TEAM_LDS_OFFSETS;
    // Grouped input whose images are all small: the checkers sort every
    // image's group order in LDS (image_sort, with the boxes and the inverse
    // permutation); the team sorts by score only, for the score order.
    bool per_image = false;
    if constexpr (GROUPED) per_image = stage_offsets(ka, sm);
    const int P = per_image ? 4 : a.passes;
    for (int j = tid; j < HIST_COPIES * Smem::DIGITS * 256; j += NT) (&sm.u.hc[0][0][0])[j] = 0u;
    const int wbase = t * S + wave * 64 * E + lane;  // element e: wbase + 64 e
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = wbase + e * 64;
        s[e] = i < n ? ka.scores[i] : 0.0f;
    }
    // the tile's boxes: finite, ordered with a positive finite area, and
    // (one image) their extent, on which the pre-test words are quantised
    bool finite = true, ordered = true;
    float4 ex = make_float4(INFINITY, INFINITY, -INFINITY, -INFINITY);
    constexpr int CH = E < 4 ? E : 4;  // boxes or ring words in flight per thread
    if (ka.boxes != nullptr) {
#pragma unroll
        for (int e0 = 0; e0 < E; e0 += CH) {
        float4 bx[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = wbase + (e0 + c) * 64;
            bx[c] = i < n ? ka.boxes[i] : make_float4(0.f, 0.f, 1.f, 1.f);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (wbase + (e0 + c) * 64 >= n) continue;
            const float4 q = bx[c];
            finite = finite && isfinite(q.x) && isfinite(q.y) && isfinite(q.z) && isfinite(q.w);
            const float ar = (q.z - q.x) * (q.w - q.y);
            ordered = ordered && q.x < q.z && q.y < q.w && ar > 0.0f && ar < INFINITY;
            ex = ext_min_max(ex, make_float4(fminf(q.x, q.z), fminf(q.y, q.w), fmaxf(q.x, q.z),
                                             fmaxf(q.y, q.w)));
        }
        }
    }
    uint32_t sk[E], ck[E], ik[E];
    uint32_t err = finite ? 0u : ERR_NONFINITE;
    if (!ordered) atomicOr(&sm.unordered, 1u);
    const bool packs = !GROUPED && ka.boxes != nullptr;
    if (packs) {
        ex = wave_ext(ex);
        if (lane == 0) sm.ext[wave] = ex;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = wbase + e * 64;
        if (s[e] != s[e] && i < n) err |= ERR_NONFINITE;
        sk[e] = score_key(s[e]);
        ck[e] = 0u;
        ik[e] = 0u;
        if constexpr (GROUPED) {
            if (i < n) {
                ck[e] = ka.class_ids ? class_key(ka.class_ids[i]) : 0u;
                ik[e] = lds_offs    ? image_in(sm.offs, ka.num_images, i)
                        : ka.offsets ? image_of(ka.offsets, ka.num_images, i)
                                     : 0u;
                st_c(&w.gcls[i], ck[e]);
                st_c(&w.gimg[i], ik[e]);
            }
        }
    }
    __syncthreads();
    {
        uint32_t(*hist)[256] = sm.u.hc[lane % HIST_COPIES];
        // A digit every valid lane of the wave shares (the high digits of a
        // score, of a small class id, of the image) is one add of the lane
        // count; others are one LDS atomic per lane.
        auto count = [&](int pos, uint32_t d, uint64_t vm, int first) {
            const uint32_t d0 = (uint32_t)__shfl((int)d, first, 64);
            if (__ballot(((vm >> lane) & 1u) && d != d0) == 0ull) {
                if (lane == first) atomicAdd(&sm.u.hc[0][pos][d0], (uint32_t)__popcll(vm));
            } else if ((vm >> lane) & 1u) {
                atomicAdd(&hist[pos][d], 1u);
            }
        };
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint64_t vm = __ballot(wbase + e * 64 < n);
            if (vm == 0ull) continue;
            const int first = __builtin_ctzll(vm);
#pragma unroll
            for (int d = 0; d < 4; ++d) count(d, (sk[e] >> (8 * d)) & 255u, vm, first);
            if constexpr (GROUPED) {
                if (P > 4) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        count(4 + d, (ck[e] >> (8 * d)) & 255u, vm, first);
                        if (8 + d < P) count(8 + d, (ik[e] >> (8 * d)) & 255u, vm, first);
                    }
                }
            }
        }
    }
    if (err) atomicOr(&sm.err, err);
    __syncthreads();
    const int cols = P * 256;
    for (int j = tid; j < cols; j += NT) {
        uint32_t sum = 0;
#pragma unroll
        for (int q = 0; q < HIST_COPIES; ++q) sum += (&sm.u.hc[q][0][0])[j];
        st_c(&tw.hist[(size_t)t * RADIX_PASSES * 256 + j], tagged(tag, sum));
    }
    if (packs && tid == 0) {
        float4 te = sm.ext[0];
        for (int v = 1; v < NW; ++v) te = ext_min_max(te, sm.ext[v]);
        uint64_t *x = tw.ext + (size_t)t * SLOT;
        st_c(&x[0], tagged(tag, __float_as_uint(te.x)));
        st_c(&x[1], tagged(tag, __float_as_uint(te.y)));
        st_c(&x[2], tagged(tag, __float_as_uint(te.z)));
        st_c(&x[3], tagged(tag, __float_as_uint(te.w)));
    }
    // Owners: member t sums the groups of 8 columns g = t, t + T, ... (a
    // group fills a 64-byte line of a tile's counts).  Lanes l and l + 32
    // hold two columns, lane l & 31 = tile; a 32-lane scan gives every
    // tile's prefix, lane 31 the total.  Four groups make a round; the loads
    // of OWNER_ROUNDS rounds are in flight together.
    bool ok = true;
    {
        constexpr int OWNER_ROUNDS = 4;
        const int tile = lane & 31;
        const int col = tid >> 5;  // 0 .. 31: four groups per round
        for (int g0 = 0; 8 * (t + T * g0) < cols; g0 += 4 * OWNER_ROUNDS) {
            // round r's column: c0 + 32 T r
            const int c0 = 8 * (t + T * (g0 + (col >> 3))) + (col & 7);
            uint32_t want = 0;
#pragma unroll
            for (int r = 0; r < OWNER_ROUNDS; ++r)
                if (c0 + 32 * T * r < cols && tile < T) want |= 1u << r;
            uint32_t v[OWNER_ROUNDS];
#pragma unroll
            for (int r = 0; r < OWNER_ROUNDS; ++r) v[r] = 0u;
            if (want && !poll_words<OWNER_ROUNDS>(
                            &tw.hist[(size_t)tile * RADIX_PASSES * 256 + c0], 32 * (size_t)T, want,
                            tag, v))
                ok = false;
#pragma unroll
            for (int r = 0; r < OWNER_ROUNDS; ++r) {
                uint32_t incl = v[r];
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) {
                    const uint32_t u = __shfl_up(incl, o, 32);
                    if (tile >= o) incl += u;
                }
                const uint32_t total = __shfl(incl, 31, 32);
                if ((want >> r) & 1u) {
                    const int c = c0 + 32 * T * r;
                    st_c(&tw.pre[(size_t)tile * RADIX_PASSES * 256 + c], tagged(tag, incl - v[r]));
                    if (tile == 0) st_c(&tw.tot[c], tagged(tag, total));
                }
            }
        }
    }
    // every member: the totals, and its own tile's prefixes
    {
        constexpr int K = (RADIX_PASSES * 256 + NT - 1) / NT;  // columns per thread at most
        uint32_t want = 0;
#pragma unroll
        for (int q = 0; q < K; ++q)
            if (tid + q * NT < cols) want |= 1u << q;
        uint32_t vt[K], vp[K];
#pragma unroll
        for (int q = 0; q < K; ++q) vt[q] = vp[q] = 0u;
        if (!poll_words<K>(&tw.tot[tid], &tw.pre[(size_t)t * RADIX_PASSES * 256 + tid], NT, want,
                           tag, vt, vp))
            ok = false;
#pragma unroll
        for (int q = 0; q < K; ++q) {
            const int j = tid + q * NT;
            if (j < cols) {
                sm.gtot[j] = vt[q];
                sm.gpre[j] = vp[q];
            }
        }
    }
    // one image: the extent of all boxes, from every member's slot
    if (packs && wave == 0) {
        float4 e4 = make_float4(INFINITY, INFINITY, -INFINITY, -INFINITY);
        if (lane < T) {
            uint32_t v[4] = {0, 0, 0, 0};
            if (!poll_words<4>(tw.ext + (size_t)lane * SLOT, 1, 0xFu, tag, v)) ok = false;
            e4 = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                             __uint_as_float(v[3]));
        }
        e4 = wave_ext(e4);
        if (lane == 0) {
            sm.ps.x0 = e4.x;
            sm.ps.y0 = e4.y;
            sm.ps.sx = pack_step(e4.x, e4.z);
            sm.ps.sy = pack_step(e4.y, e4.w);
        }
    }
    if (!ok) atomicOr(&sm.err, ERR_INTERNAL);
    __syncthreads();
    // the plan: a pass whose digit is the same for every key moves nothing
    if (wave < P) {
        const uint32_t un = (uint32_t)n;
        const uint32_t *g = &sm.gtot[wave * 256];
        const bool one = g[4 * lane] == un || g[4 * lane + 1] == un || g[4 * lane + 2] == un ||
                         g[4 * lane + 3] == un;
        const uint64_t any = __ballot(one);
        if (lane == 0) sm.skip[wave] = any ? 1u : 0u;
    }
    __syncthreads();
    int last = -1, last_score = -1;
    for (int p = 0; p < P; ++p)
        if (!sm.skip[p]) {
            last = p;
            if (p < 4) last_score = p;
        }
    // every key the same: the last pass runs anyway (it moves nothing) and
    // writes the outputs
    if (last < 0) last = P - 1;
    if (tid == 0) {
        int m = 0;
        for (int p = 0; p < P; ++p)
            if (!sm.skip[p] || p == last) sm.act[m++] = p;
        sm.nact = m;
    }
    if (GROUPED && last_score < 0) {
        // no score pass moves anything: the score order is the input order
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = wbase + e * 64;
            if (i < n) w.score_order[i] = i;
        }
    }

    // ---------------------------------------------------------- passes
    __syncthreads();
    const int count = n - t * S < S ? n - t * S : S;
    const int nact = sm.nact;
    const size_t ring_words = 2 * (size_t)ka.npad;
    uint32_t k[E], v[E], rk[E];
    for (int j = 0; j < nact; ++j) {
        const int p = sm.act[j];
        const int shift = 8 * (p & 3);
        const int kind = p >> 2;  // 0 score, 1 class, 2 image
        const bool is_last = j == nact - 1;
        // the tile's values and keys: the first pass keeps phase 0's; later
        // ones load the ring words of their positions once they carry this
        // pass's tag (no barrier: each word says whether it is written)
        if (j == 0) {
            // (a first pass on the class or the image, every score digit
            // being shared, looks its keys up again rather than keep them)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int i = wbase + e * 64;
                v[e] = (uint32_t)i;
                k[e] = sk[e];
                if (GROUPED && kind != 0 && i < n) {
                    if (kind == 1) k[e] = ka.class_ids ? class_key(ka.class_ids[i]) : 0u;
                    else k[e] = lds_offs    ? image_in(sm.offs, ka.num_images, i)
                                : ka.offsets ? image_of(ka.offsets, ka.num_images, i)
                                             : 0u;
                }
            }
        } else {
            const uint64_t *rb = a.ring + (size_t)(j % 3) * ring_words + 2 * (size_t)wbase;
            uint32_t want = 0;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (wbase + e * 64 < n) want |= 1u << e;
#pragma unroll
            for (int e0 = 0; e0 < E; e0 += CH) {
                uint32_t cv[CH], ck2[CH];
#pragma unroll
                for (int c = 0; c < CH; ++c) cv[c] = ck2[c] = 0u;
                if (!poll_words<CH>(rb + 128 * e0, rb + 128 * e0 + 1, 128,
                                    (want >> e0) & ((1u << CH) - 1u), ring_tag(a.epoch, j), cv,
                                    ck2))
                    atomicOr(&sm.err, ERR_INTERNAL);
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    v[e0 + c] = cv[c];
                    k[e0 + c] = ck2[c];
                }
            }
            // The values are input indices.  Only after a wait gave up could
            // one be out of range; it is then replaced, and the call reports
            // ERR_INTERNAL.
            bool bad = false;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (v[e] >= (uint32_t)n) {
                    bad = true;
                    v[e] = 0u;
                }
            }
            if (bad) atomicOr(&sm.err, ERR_INTERNAL);
        }
        // rank the tile
        {
            uint32_t dg[E];
#pragma unroll
            for (int e = 0; e < E; ++e) dg[e] = (k[e] >> shift) & 255u;
            rank_digits<E>(sm, dg, count, rk);
        }
        __syncthreads();
        if (tid < 256) {
            const int d = tid;
            uint32_t run = 0;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                const uint32_t c = sm.wcnt[wv][d];
                sm.wpre[wv][d] = run;
                run += c;
            }
            sm.tcnt[d] = run;
            if (j > 0) st_c(&tw.cnt[((size_t)p * tw.tl + t) * 256 + d], tagged(tag, run));
        }
        if (wave == 0) scan256(&sm.gtot[p * 256], sm.gb);
        __syncthreads();
        // the tile's offset per digit among the earlier tiles
        if (j == 0) {
            if (tid < 256) sm.part[0][tid] = sm.gpre[p * 256 + tid];
        } else {
            // thread (q, d) sums the counts of tiles q, q + 4, ... below t
            const int d = tid & 255, q = tid >> 8;
            constexpr int KT = TEAM_MAX / 4;
            uint32_t want = 0;
#pragma unroll
            for (int m = 0; m < KT; ++m)
                if (q + 4 * m < t) want |= 1u << m;
            uint32_t c[KT];
#pragma unroll
            for (int m = 0; m < KT; ++m) c[m] = 0;
            if (want && !poll_words<KT>(&tw.cnt[((size_t)p * tw.tl + q) * 256 + d], 4 * 256, want,
                                        tag, c))
                atomicOr(&sm.err, ERR_INTERNAL);
            uint32_t sum = 0;
#pragma unroll
            for (int m = 0; m < KT; ++m) sum += c[m];
            sm.part[q][d] = sum;
        }
        if (wave == 0) scan256(sm.tcnt, sm.tbase);
        __syncthreads();
        if (tid < 256) {
            uint32_t ex = sm.part[0][tid];
            if (j > 0) ex += sm.part[1][tid] + sm.part[2][tid] + sm.part[3][tid];
            sm.gsh[tid] = (int32_t)(sm.gb[tid] + ex) - (int32_t)sm.tbase[tid];
        }
        // reorder the tile by digit in LDS
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (wbase + e * 64 < n) {
                const uint32_t d = (k[e] >> shift) & 255u;
                const uint32_t slot = sm.tbase[d] + sm.wpre[wave][d] + rk[e];
                sm.u.stage.k[slot] = k[e];
                sm.u.stage.v[slot] = v[e];
            }
        }
        // The ring this pass writes was last read by pass j - 2: every
        // member must have loaded that pass's tile, which its counts for
        // that pass (published after the loads) show.
        if (j >= 3 && !is_last && wave == 0) {
            const int pr = sm.act[j - 2];
            for (int tt = lane; tt < T; tt += 64) {
                uint32_t c[1] = {0};
                if (!poll_words<1>(&tw.cnt[((size_t)pr * tw.tl + tt) * 256], 0, 1u, tag, c))
                    atomicOr(&sm.err, ERR_INTERNAL);
            }
        }
        __syncthreads();
        const bool score_order_here = GROUPED && p == last_score;
        if (!is_last) {
            // the next pass's key: the same key, or at a change of kind the
            // class key or the image of the box
            const int nk = sm.act[j + 1] >> 2;
            uint64_t *wb = a.ring + (size_t)((j + 1) % 3) * ring_words;
            const uint32_t tag_out = ring_tag(a.epoch, j + 1);
            bool bad = false;
            for (int s0 = tid; s0 < count; s0 += NT) {
                const uint32_t key = sm.u.stage.k[s0];
                const int pos = s0 + sm.gsh[(key >> shift) & 255u];
                const uint32_t val = sm.u.stage.v[s0];
                // in range unless a wait gave up (see above)
                if ((uint32_t)pos >= (uint32_t)n) {
                    bad = true;
                    continue;
                }
                uint32_t nkey = key;
                if (GROUPED && nk != kind) {
                    if (nk == 1) nkey = ka.class_ids ? class_key(ka.class_ids[val]) : 0u;
                    else nkey = lds_offs    ? image_in(sm.offs, ka.num_images, val)
                                : ka.offsets ? image_of(ka.offsets, ka.num_images, val)
                                             : 0u;
                }
                if (score_order_here) w.score_order[pos] = (int32_t)val;
                st_c(&wb[2 * (size_t)pos], tagged(tag_out, val));
                st_c(&wb[2 * (size_t)pos + 1], tagged(tag_out, nkey));
            }
            if (bad) atomicOr(&sm.err, ERR_INTERNAL);
        } else {
            const PackScale ps = sm.ps;
            // The sorted order, and (boxes given: the sort-only export passes
            // none) the sorted boxes with their areas.  All of a thread's box
            // loads are issued before any of its stores.
#pragma unroll
            for (int q0 = 0; q0 < E; q0 += CH) {
            int pos[CH];
            uint32_t val[CH];
            float4 bx[CH];
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                const int s0 = tid + (q0 + q) * NT;
                pos[q] = -1;
                val[q] = 0u;
                if (s0 < count) {
                    const uint32_t key = sm.u.stage.k[s0];
                    const int pq = s0 + sm.gsh[(key >> shift) & 255u];
                    // in range unless a wait gave up (see above)
                    if ((uint32_t)pq < (uint32_t)n) {
                        pos[q] = pq;
                        val[q] = sm.u.stage.v[s0];
                    } else {
                        atomicOr(&sm.err, ERR_INTERNAL);
                    }
                }
                bx[q] = ka.boxes != nullptr && pos[q] >= 0 ? ka.boxes[val[q]]
                                                           : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                if (pos[q] < 0) continue;
                if (score_order_here) w.score_order[pos[q]] = (int32_t)val[q];
                if (per_image) continue;  // the checkers write the group order
                w.order[pos[q]] = (int32_t)val[q];
                if (GROUPED) w.inv[val[q]] = pos[q];
                if (ka.boxes == nullptr) continue;
                const float4 bj = bx[q];
                w.sb[pos[q]] = bj;
                w.area[pos[q]] = (bj.z - bj.x) * (bj.w - bj.y);
                if (packs) {
                    const uint2 crs = coarse_words(bj, ps);
                    w.scol[pos[q]] = crs.x;
                    w.srow[pos[q]] = crs.y;
                }
            }
            }
        }
        // the next pass rewrites the staged tile and the counts
        __syncthreads();
    }

    // ---------------------------------------------------------- report
    __syncthreads();
    if (tid == 0)
        st_c(&tw.done[(size_t)t * SLOT],
             tagged(tag, sm.err | (sm.unordered ? UNORDERED_BIT : 0u)));
    if (t != 0) return;
    // member 0: every member's and every checker's bits, then the control
    // block
    if (tid == 0) sm.part[0][0] = 0u;
    __syncthreads();
    for (int j = tid; j < T + a.checkers; j += NT) {
        uint32_t out[1] = {0};
        if (!poll_words<1>(j < T ? &tw.done[(size_t)j * SLOT] : &tw.chk[(size_t)(j - T) * SLOT],
                           0, 1u, tag, out))
            out[0] = ERR_INTERNAL;
        if (out[0]) atomicOr(&sm.part[0][0], out[0]);
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t all = sm.part[0][0];
        Ctrl *c = w.ctrl;
        c->error = all & ~UNORDERED_BIT;
        c->flags = (all & UNORDERED_BIT) ? 0u : FLAG_ORDERED_BOXES;
        c->count = 0;
        c->num_items = GROUPED ? 0 : item_base_full(ka.words, ka.words, ka.strip);
        c->band_stride = ka.mstride;
        c->num_segments = 1;
        c->sweep_done = 0u;
    }
}

// ------------------------------------------------------------ sample sort
//
// One image, in one launch, by sample sort: the same stable order as the
// radix passes (score key ascending, i.e. score descending, equal scores in
// input order: "LeetCUDA 14-nms", algorithm and data flow, step 1), with
// three hand-overs between workgroups instead of one per radix pass plus
// the counting round.
//
//   samples   member t keys its tile, checks its boxes and publishes their
//             extent and the keys of SAMPLE_PER_MEMBER evenly spaced boxes
//             (sample q is box q * stride, so its index needs no word).
//   buckets   every member reads all samples (at most 512, one per
//             thread), sorts them in LDS (stable by key, so equal keys stay
//             in index order) and takes 255 of them as splitters, (key,
//             index) pairs in that order.  A box's bucket
//             is the number of splitters at or below its (key, index); the
//             buckets are ranges of the final order.  The member ranks its
//             tile by bucket (stable), publishes the tile's bucket counts,
//             reads every tile's counts (its prefix among the tiles before
//             it, and the totals) and writes each box's (index, key) at its
//             bucket's start + prefix + rank, the tile staged in bucket order
//             in LDS so that each bucket's share goes out as one run.  Member
//             0 publishes the totals.
//   sort      every workgroup (members after their tile, the rest after their
//             share of the per-call initialisation) takes buckets b, b +
//             blocks, ...: it reads the bucket's boxes, sorts them in LDS by
//             key (stable: they arrive in index order) and writes the sorted
//             order, boxes, areas and pre-test words at the bucket's place.
//
// A bucket larger than the LDS holds (an input whose sampled boxes misjudge
// the distribution badly) is not sorted: the call raises FLAG_SORT_RETRY and
// the host runs it again with the radix passes.  Words carry the call's tags
// as in the radix passes; every wait is bounded.

constexpr int SAMPLE_PER_MEMBER = 16;   // samples per member tile
constexpr int BUCKETS = 256;
constexpr int SORT_CAP = 4096;           // boxes one workgroup sorts in LDS
// member's report word: a bucket was too large
constexpr uint32_t RETRY_BIT = 0x40000000u;

struct SampleSmem {
    struct Lds {
        uint32_t key[SORT_CAP];
        uint32_t val[SORT_CAP];
        uint32_t perm[2][SORT_CAP];
    } s;
    uint32_t gtot[4 * 256];  // digit counts of an LDS sort
    uint32_t wcnt[NW][256];
    uint32_t wpre[NW][256];
    uint32_t tcnt[256];
    uint32_t tbase[256];
    uint32_t gb[BUCKETS];     // bucket starts
    uint32_t tot[BUCKETS];    // bucket sizes
    int32_t gsh[BUCKETS];     // output position minus staged slot, per bucket
    uint32_t part[8][256];    // look-back partial sums
    uint64_t spl[BUCKETS];    // splitters (key << 32 | index); [0] unused
    float4 ext[NW];
    PackScale ps;
    uint32_t varying;  // bits in which some key differs from the first
    uint32_t err, unordered;
};

// OR over the lanes of the wave (DPP steps; lane 63 holds the result).
__device__ __forceinline__ uint32_t wave_or_to_63(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// Stable sort of positions 0 .. cnt - 1 (cnt <= EI * NT) of sm.s.key by
// key: 8-bit LSD passes, skipping a digit every key shares (found as the
// bits in which no key differs from the first).  Returns the perm buffer
// holding the sorted positions.
template <int EI>
__device__ int lds_sort(SampleSmem &sm, int cnt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto &s = sm.s;
    // the digits every key shares (those of the first key) need no pass
    if (tid == 0) sm.varying = 0u;
    __syncthreads();
    const uint32_t k0 = s.key[0];
    uint32_t dif = 0u;
#pragma unroll
    for (int e = 0; e < EI; ++e) {
        const int v = e * NT + tid;
        if (v < cnt) {
            s.perm[0][v] = (uint32_t)v;
            dif |= s.key[v] ^ k0;
        }
    }
    dif = wave_or_to_63(dif);
    if (lane == 63 && dif) atomicOr(&sm.varying, dif);
    __syncthreads();
    const uint32_t varying = sm.varying;
    const int nwa = min(NW, (cnt + 64 * EI - 1) / (64 * EI));
    int cur = 0;
    for (int q = 0; q < 4; ++q) {
        if (((varying >> (8 * q)) & 255u) == 0u) continue;
        const int shift = 8 * q;
        uint32_t v[EI], d[EI], rk[EI];
#pragma unroll
        for (int e = 0; e < EI; ++e) {
            const int i = wave * 64 * EI + e * 64 + lane;
            v[e] = i < cnt ? s.perm[cur][i] : 0u;
            d[e] = i < cnt ? (s.key[v[e]] >> shift) & 255u : 0u;
        }
        rank_digits<EI>(sm, d, cnt, rk);
        __syncthreads();
        if (wave == 0) digit_slots(sm, nwa);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EI; ++e)
            if (wave * 64 * EI + e * 64 + lane < cnt)
                s.perm[cur ^ 1][sm.wpre[wave][d[e]] + rk[e]] = v[e];
        __syncthreads();
        cur ^= 1;
    }
    return cur;
}

template <int E>
__global__ __launch_bounds__(NT) void team_sample_kernel(TeamArgs a) {
    constexpr int S = E * NT;
    constexpr int STRIDE = S / SAMPLE_PER_MEMBER;
    static_assert(STRIDE * SAMPLE_PER_MEMBER == S && TEAM_MAX * SAMPLE_PER_MEMBER <= NT,
                  "every sample is one thread's in the LDS sort");
    __shared__ SampleSmem sm;
    const KeysArgs &ka = a.ka;
    const Work &w = ka.w;
    const TeamWork tw = team_work(a.team_ws, a.tl);
    const uint32_t tag = (uint32_t)a.epoch;
    const uint32_t tag_s = ring_tag(a.epoch, 0), tag_b = ring_tag(a.epoch, 1);
    const int b = blockIdx.x, nb = (int)gridDim.x;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int T = a.team, n = ka.n;
    const size_t ring_words = 2 * (size_t)ka.npad;
    uint64_t *samples = a.ring;               // [ns]: tagged keys
    uint64_t *bkt = a.ring + ring_words;      // [2 n]: (index, key) at each position
    const int ns = (n + STRIDE - 1) / STRIDE;  // sample q is box q * STRIDE
    if (tid == 0) {
        sm.err = 0u;
        sm.unordered = 0u;
    }
    __syncthreads();
    bool ok = true;
    // a checker's share of the per-call initialisation (members, which do
    // none when there are checkers, go straight to their tile)
    if (b >= T || a.checkers == 0) {
        const uint32_t e = team_check<false>(a, b >= T ? b - T : b, a.checkers ? a.checkers : T);
        if (e) atomicOr(&sm.err, e);
    }
    if (b < T) {
        const int t = b;
        // ------------------------------------------------------ samples
        const int wbase = t * S + wave * 64 * E + lane;  // element e: wbase + 64 e
        float s[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = wbase + e * 64;
            s[e] = i < n ? ka.scores[i] : 0.0f;
        }
        bool finite = true, ordered = true;
        float4 ex = make_float4(INFINITY, INFINITY, -INFINITY, -INFINITY);
        constexpr int CH = E < 4 ? E : 4;
        if (ka.boxes != nullptr) {
#pragma unroll
            for (int e0 = 0; e0 < E; e0 += CH) {
                float4 bx[CH];
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int i = wbase + (e0 + c) * 64;
                    bx[c] = i < n ? ka.boxes[i] : make_float4(0.f, 0.f, 1.f, 1.f);
                }
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    if (wbase + (e0 + c) * 64 >= n) continue;
                    const float4 q = bx[c];
                    finite = finite && isfinite(q.x) && isfinite(q.y) && isfinite(q.z) &&
                             isfinite(q.w);
                    const float ar = (q.z - q.x) * (q.w - q.y);
                    ordered = ordered && q.x < q.z && q.y < q.w && ar > 0.0f && ar < INFINITY;
                    ex = ext_min_max(ex, make_float4(fminf(q.x, q.z), fminf(q.y, q.w),
                                                     fmaxf(q.x, q.z), fmaxf(q.y, q.w)));
                }
            }
        }
        uint32_t sk[E];
        uint32_t err = finite ? 0u : ERR_NONFINITE;
        if (!ordered) atomicOr(&sm.unordered, 1u);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = wbase + e * 64;
            if (s[e] != s[e] && i < n) err |= ERR_NONFINITE;
            sk[e] = score_key(s[e]);
            if (i < n && i % STRIDE == 0) st_c(&samples[i / STRIDE], tagged(tag_s, sk[e]));
        }
        if (err) atomicOr(&sm.err, err);
        const bool packs = ka.boxes != nullptr;
        if (packs) {
            ex = wave_ext(ex);
            if (lane == 0) sm.ext[wave] = ex;
        }
        __syncthreads();
        if (packs && tid == 0) {
            float4 te = sm.ext[0];
            for (int v = 1; v < NW; ++v) te = ext_min_max(te, sm.ext[v]);
            uint64_t *x = tw.ext + (size_t)t * SLOT;
            st_c(&x[0], tagged(tag, __float_as_uint(te.x)));
            st_c(&x[1], tagged(tag, __float_as_uint(te.y)));
            st_c(&x[2], tagged(tag, __float_as_uint(te.z)));
            st_c(&x[3], tagged(tag, __float_as_uint(te.w)));
        }
        // ------------------------------------------------------ buckets
        // every sample (in index order), sorted by key
        {
            uint32_t v[1] = {0u};
            if (tid < ns && !poll_words<1>(&samples[tid], 0, 1u, tag_s, v)) ok = false;
            if (tid < ns) sm.s.key[tid] = v[0];
        }
        __syncthreads();
        const int sc = lds_sort<1>(sm, ns);
        // splitter j (1 .. 255): the sample of sorted rank j * ns / 256
        if (tid > 0 && tid < BUCKETS) {
            const uint32_t q = sm.s.perm[sc][(int)(((int64_t)tid * ns) / BUCKETS)];
            sm.spl[tid] = ((uint64_t)sm.s.key[q] << 32) | (uint64_t)(q * (uint32_t)STRIDE);
        }
        __syncthreads();
        // each box's bucket: the splitters at or below its (key, index)
        uint32_t bk[E], rk[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = wbase + e * 64;
            const uint64_t x = ((uint64_t)sk[e] << 32) | (uint64_t)(uint32_t)i;
            uint32_t lo = 0;
#pragma unroll
            for (int step = BUCKETS / 2; step > 0; step >>= 1)
                if (sm.spl[lo + step] <= x) lo += step;
            bk[e] = i < n ? lo : 0u;
        }
        const int count = n - t * S < S ? n - t * S : S;
        rank_digits<E>(sm, bk, count, rk);
        __syncthreads();
        if (tid < 256) {
            uint32_t run = 0;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                const uint32_t c = sm.wcnt[wv][tid];
                sm.wpre[wv][tid] = run;
                run += c;
            }
            sm.gtot[tid] = run;  // this tile's count of each bucket
            st_c(&tw.cnt[(size_t)t * 256 + tid], tagged(tag, run));
        }
        // every tile's counts: thread (q, d) sums tiles q, q + 4, ...,
        // those before t apart
        {
            const int d = tid & 255, q = tid >> 8;
            constexpr int KT = TEAM_MAX / 4;
            uint32_t want = 0;
#pragma unroll
            for (int m = 0; m < KT; ++m)
                if (q + 4 * m < T) want |= 1u << m;
            uint32_t c[KT];
#pragma unroll
            for (int m = 0; m < KT; ++m) c[m] = 0;
            if (want && !poll_words<KT>(&tw.cnt[(size_t)q * 256 + d], 4 * 256, want, tag, c))
                ok = false;
            uint32_t before = 0, all = 0;
#pragma unroll
            for (int m = 0; m < KT; ++m) {
                all += c[m];
                if (q + 4 * m < t) before += c[m];
            }
            sm.part[q][d] = before;
            sm.part[4 + q][d] = all;
        }
        __syncthreads();
        if (tid < 256) {
            const uint32_t all = sm.part[4][tid] + sm.part[5][tid] + sm.part[6][tid] +
                                 sm.part[7][tid];
            sm.tot[tid] = all;
            sm.tcnt[tid] = sm.part[0][tid] + sm.part[1][tid] + sm.part[2][tid] + sm.part[3][tid];
            if (t == 0) st_c(&tw.tot[tid], tagged(tag, all));
        }
        __syncthreads();
        if (wave == 0) scan256(sm.tot, sm.gb);
        if (wave == 1) scan256(sm.gtot, sm.tbase);
        __syncthreads();
        // The tile in bucket order through LDS, so that each bucket's boxes
        // go out as one run: a box lands at its bucket's start + the boxes of
        // its bucket in the tiles before + its rank in this tile.
        if (tid < 256)
            sm.gsh[tid] = (int32_t)(sm.gb[tid] + sm.tcnt[tid]) - (int32_t)sm.tbase[tid];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (wbase + e * 64 >= n) continue;
            const uint32_t d = bk[e];
            const uint32_t slot = sm.tbase[d] + sm.wpre[wave][d] + rk[e];
            sm.s.key[slot] = sk[e];
            sm.s.val[slot] = (uint32_t)(wbase + e * 64);
            sm.s.perm[0][slot] = d;
        }
        __syncthreads();
        for (int s0 = tid; s0 < count; s0 += NT) {
            const int pos = s0 + sm.gsh[sm.s.perm[0][s0]];
            if ((uint32_t)pos >= (uint32_t)n) {
                ok = false;  // only after a wait gave up
                continue;
            }
            st_c(&bkt[2 * (size_t)pos], tagged(tag_b, sm.s.val[s0]));
            st_c(&bkt[2 * (size_t)pos + 1], tagged(tag_b, sm.s.key[s0]));
        }
        __syncthreads();  // the LDS sort below reuses the arrays
    }

    // ---------------------------------------------------------- sort
    // the bucket sizes, and (boxes given) the extent of all boxes
    {
        uint32_t v[1] = {0};
        if (tid < BUCKETS && !poll_words<1>(&tw.tot[tid], 0, 1u, tag, v)) ok = false;
        if (tid < BUCKETS) sm.tot[tid] = v[0];
    }
    if (ka.boxes != nullptr && wave == 0) {
        float4 e4 = make_float4(INFINITY, INFINITY, -INFINITY, -INFINITY);
        if (lane < T) {
            uint32_t v[4] = {0, 0, 0, 0};
            if (!poll_words<4>(tw.ext + (size_t)lane * SLOT, 1, 0xFu, tag, v)) ok = false;
            e4 = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                             __uint_as_float(v[3]));
        }
        e4 = wave_ext(e4);
        if (lane == 0) {
            sm.ps.x0 = e4.x;
            sm.ps.y0 = e4.y;
            sm.ps.sx = pack_step(e4.x, e4.z);
            sm.ps.sy = pack_step(e4.y, e4.w);
        }
    }
    __syncthreads();
    if (wave == 0) scan256(sm.tot, sm.gb);
    __syncthreads();
    bool retry = false;
    for (int bu = b; bu < BUCKETS; bu += nb) {
        const int cnt = (int)sm.tot[bu];
        const uint32_t start = sm.gb[bu];
        if (cnt == 0) continue;
        if (cnt > SORT_CAP || start + (uint32_t)cnt > (uint32_t)n) {
            retry = true;
            continue;
        }
        {
            constexpr int K = SORT_CAP / NT;
            uint32_t want = 0;
#pragma unroll
            for (int m = 0; m < K; ++m)
                if (tid + m * NT < cnt) want |= 1u << m;
            uint32_t vi[K], vk[K];
#pragma unroll
            for (int m = 0; m < K; ++m) vi[m] = vk[m] = 0u;
            const uint64_t *p = bkt + 2 * ((size_t)start + tid);
            if (!poll_words<K>(p, p + 1, 2 * (size_t)NT, want, tag_b, vi, vk)) ok = false;
#pragma unroll
            for (int m = 0; m < K; ++m) {
                const int r = tid + m * NT;
                if (r < cnt) {
                    // an index out of range only after a wait gave up
                    sm.s.val[r] = vi[m] < (uint32_t)n ? vi[m] : 0u;
                    sm.s.key[r] = vk[m];
                }
            }
        }
        __syncthreads();
        const int cur = cnt <= NT       ? lds_sort<1>(sm, cnt)
                        : cnt <= 2 * NT ? lds_sort<2>(sm, cnt)
                                        : lds_sort<SORT_CAP / NT>(sm, cnt);
        const PackScale ps = sm.ps;
        for (int r = tid; r < cnt; r += NT) {
            const int pos = (int)start + r;
            const int i = (int)sm.s.val[sm.s.perm[cur][r]];
            w.order[pos] = i;
            if (ka.boxes != nullptr) {
                const float4 bj = ka.boxes[i];
                w.sb[pos] = bj;
                w.area[pos] = (bj.z - bj.x) * (bj.w - bj.y);
                const uint2 crs = coarse_words(bj, ps);
                w.scol[pos] = crs.x;
                w.srow[pos] = crs.y;
            }
        }
        __syncthreads();  // the next bucket reuses the LDS
    }
    if (!ok) atomicOr(&sm.err, ERR_INTERNAL);
    __syncthreads();
    // ---------------------------------------------------------- report
    const uint32_t mine = sm.err | (sm.unordered ? UNORDERED_BIT : 0u) | (retry ? RETRY_BIT : 0u);
    if (b >= T) {
        if (tid == 0) st_c(&tw.chk[(size_t)(b - T) * SLOT], tagged(tag, mine));
        return;
    }
    // (retry is the same in every thread of a block: a block-wide property)
    if (tid == 0) st_c(&tw.done[(size_t)b * SLOT], tagged(tag, mine));
    if (b != 0) return;
    if (tid == 0) sm.part[0][0] = 0u;
    __syncthreads();
    for (int j = tid; j < T + a.checkers; j += NT) {
        uint32_t out[1] = {0};
        if (!poll_words<1>(j < T ? &tw.done[(size_t)j * SLOT] : &tw.chk[(size_t)(j - T) * SLOT],
                           0, 1u, tag, out))
            out[0] = ERR_INTERNAL;
        if (out[0]) atomicOr(&sm.part[0][0], out[0]);
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t all = sm.part[0][0];
        Ctrl *c = w.ctrl;
        c->error = all & ~(UNORDERED_BIT | RETRY_BIT);
        c->flags = ((all & UNORDERED_BIT) ? 0u : FLAG_ORDERED_BOXES) |
                   ((all & RETRY_BIT) ? FLAG_SORT_RETRY : 0u);
        c->count = 0;
        c->num_items = item_base_full(ka.words, ka.words, ka.strip);
        c->band_stride = ka.mstride;
        c->num_segments = 1;
        c->sweep_done = 0u;
    }
}

// Elements per thread of a team of at most tmax members (tiles of e * NT
// boxes) for n boxes; 0 when n is too large.
int team_elems(int64_t n, int tmax) {
    for (int e = 1; e <= TEAM_EMAX; e *= 2)
        if ((n + (int64_t)e * NT - 1) / ((int64_t)e * NT) <= tmax) return e;
    return 0;
}

// XCDs of the current device (cached per device; 1 when unknown).
int device_xcc_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    if (cached[dev] == 0) {
        int x = 0;
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x <= 0)
            x = 1;
        cached[dev] = x;
    }
    return cached[dev];
}

struct TeamShape {
    int e, team, blocks;
};

// The team's shape on the current device: members are blocks 0 .. T - 1,
// at most TEAM_MAX and at most one per XCD's worth of compute units, so that
// every member is resident (one workgroup per compute unit); blocks T .. up
// to T * (XCDs, at most 8) check.
TeamShape team_shape(int64_t n) {
    TeamShape s{0, 0, 0};
    int xcc = device_xcc_count();
    xcc = xcc < 1 ? 1 : (xcc > 8 ? 8 : xcc);
    const int per_xcd = device_cu_count() / xcc;
    const int tmax = per_xcd < TEAM_MAX ? per_xcd : TEAM_MAX;
    if (tmax < 1 || n < 1) return s;
    s.e = team_elems(n, tmax);
    if (s.e > 0) {
        s.team = (int)((n + (int64_t)s.e * NT - 1) / ((int64_t)s.e * NT));
        s.blocks = s.team * xcc;
    }
    return s;
}

}  // namespace

bool team_sample_applies(const Problem &P) {
    if (P.grouped || P.n <= RANK_SORT_MAX || P.n > TEAM_MAX_N) return false;
    return team_shape(P.n).team > 0;
}

bool team_sort_applies(const Problem &P) {
    if (P.n < 1 || P.n > TEAM_MAX_N) return false;
    if (!P.grouped && P.n <= RANK_SORT_MAX) return false;
    return team_shape(P.n).team > 0;
}

namespace {

// The launch's arguments; false when the workspace lacks the team's words.
bool team_args(const Problem &P, const Layout &L, const Work &w, uint64_t epoch,
               const TeamShape &s, TeamArgs &a) {
    const int tl = (int)team_layout_members(P.n);
    if (s.team <= 0 || s.team > tl || L.off_team == 0 || w.team == nullptr) return false;
    // the carve must end where the layout's region ends
    const TeamWork tw = team_work(w.team, tl);
    if ((size_t)(tw.end - w.team) * 8 != team_ws_bytes(tl)) return false;
    KeysArgs &ka = a.ka;
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
    ka.tiles = s.team;
    ka.grouped = P.grouped ? 1 : 0;
    ka.w = w;
    a.team = s.team;
    a.checkers = s.blocks - s.team;
    int image_digits = 0;
    for (int64_t m = (int64_t)P.num_images - 1; m > 0; m >>= 8) ++image_digits;
    a.passes = P.grouped ? 8 + image_digits : 4;
    a.epoch = epoch;
    a.team_ws = w.team;
    a.tl = tl;
    a.ring = w.team_ring;
    return a.ring != nullptr;
}

}  // namespace

hipError_t launch_team_sort(const Problem &P, const Layout &L, const Work &w, uint64_t epoch,
                            hipStream_t stream) {
    const TeamShape s = team_shape(P.n);
    TeamArgs a;
    if (!team_args(P, L, w, epoch, s, a)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)s.blocks), block(NT);
#define GNMS_TEAM_LAUNCH(EV)                                                         \
    if (s.e == EV) {                                                                 \
        if (P.grouped)                                                               \
            hipLaunchKernelGGL((team_sort_kernel<EV, true>), grid, block, 0, stream, a); \
        else                                                                         \
            hipLaunchKernelGGL((team_sort_kernel<EV, false>), grid, block, 0, stream, a); \
    }
    GNMS_TEAM_LAUNCH(1)
    GNMS_TEAM_LAUNCH(2)
    GNMS_TEAM_LAUNCH(4)
#undef GNMS_TEAM_LAUNCH
    return hipGetLastError();
}

hipError_t launch_team_sample(const Problem &P, const Layout &L, const Work &w, uint64_t epoch,
                              hipStream_t stream) {
    const TeamShape s = team_shape(P.n);
    TeamArgs a;
    if (P.grouped || !team_args(P, L, w, epoch, s, a)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)s.blocks), block(NT);
    if (s.e == 1) hipLaunchKernelGGL(team_sample_kernel<1>, grid, block, 0, stream, a);
    if (s.e == 2) hipLaunchKernelGGL(team_sample_kernel<2>, grid, block, 0, stream, a);
    if (s.e == 4) hipLaunchKernelGGL(team_sample_kernel<4>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace gnms
