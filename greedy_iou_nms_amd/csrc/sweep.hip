// Stages (c) and (d): the greedy sweep over the suppression bitmask, then the
// compaction that maps kept sorted positions back to input indices.
//
// Sweep ("LeetCUDA 14-nms", Phase 2).  The removed bitmap (one bit per sorted
// box, W = ceil(n/64) words) lives in LDS and the boxes are visited in score
// order, 64 at a time (one row tile, "chunk" c).  Settling chunk c needs the
// removed word c complete, i.e. every kept row before the chunk ORed in.  A
// row's words for the next few tiles are needed soon; words far to the right
// of it can be ORed in any time before the sweep gets there.  The workgroup
// is split accordingly:
//   * the resolver (wave 0) walks the chunks in order.  Lane k holds the
//     diagonal word M[64c + k][c]; the chunk is settled serially in scalar
//     registers: the lowest not-yet-removed row k whose diagonal word is
//     nonzero is kept and ORs its word in; rows whose diagonal word is zero
//     remove nothing inside the chunk, so only rows that survive and suppress
//     cost a step; every row still clear at the end is kept.  It publishes
//     the kept set and ORs the kept rows' words for the next NEAR tiles into
//     words c + 1 .. c + NEAR itself.
//   * appliers (waves 1..7) own every 7th chunk.  Long before the resolver
//     gets there, an applier loads its chunk's diagonal and near words
//     (which it stages in LDS for the resolver), the row tile's count of
//     nonzero words and then the tile's list of them (row, word, value)
//     written by the mask kernel; when the kept set is published it ORs the
//     kept rows' words for column tiles c + NEAR + 1 and later into the
//     bitmap.  A tile whose list overflowed has its kept rows read densely.
//     For one image the applier also writes the chunk's kept boxes to the
//     output: the resolver hands over, with the kept set, the number of
//     boxes kept before the chunk, and each kept lane stores order[64c +
//     lane] at that offset plus its rank in the chunk.  The output is thus
//     complete when the last chunk is applied.
// The resolver waits for chunk c - NEAR - 1 to be applied before it reads
// word c, so an applier has NEAR chunk settlements of slack.
// The page's sweep takes one barrier per box; here no barrier is taken: the
// waves hand chunks over through LDS flags (release/acquire at workgroup
// scope), and every wait is bounded -- a wait that gives up raises an
// internal error and all waves leave, so no configuration can hang the GPU.
// A box is kept iff its removed bit is clear when the sweep reaches it, and
// later rows never set bits at or below their own position, so the kept set
// is the complement of the final bitmap.
//
// Compaction (the page's host-side map-back, bug 3, done on the device).  For
// one image the sorted order is the score order and the appliers write the
// kept boxes' input indices order[p] as int64 while the sweep runs (above).
// For grouped input the kept bits are in group order; the compaction kernel
// walks the plain score order and looks each box's sorted position up
// through the inverse permutation, so the output is one list in global score
// order.
#include "mask_core.h"
#include "nms_internal.h"
#include "rank_core.h"

namespace gnms {
namespace {

constexpr int NT = SWEEP_THREADS;
constexpr int NWAVES = NT / 64;

struct SweepArgs {
    const uint64_t *mask;
    const int32_t *tile_cend;
    const int32_t *order;
    const uint32_t *tcount;
    const uint32_t *tent_wk;
    const uint64_t *tent_val;
    const uint64_t *tnear;
    Ctrl *ctrl;
    uint64_t *kept;
    int64_t *keep_out;
    // fused with the mask: per row tile, mask work items finished
    const uint32_t *done;
    int n, words, npad, mstride, strip, grouped;
    int strip_groups;  // ceil(W / strip): mask work pairs of row tile 0
    int done_shift;    // fused: a finished pair adds 64 << done_shift to done[]
    int dense;         // the mask kernel wrote dense rows (see Problem::dense)
    Post post;         // the call's result, when this sweep ends the call
};

// Reads of data the mask stage writes.  In the fused kernel the mask is still
// running on other XCDs, so they are device-scope (coherent) loads.
template <bool FUSED, typename T>
__device__ __forceinline__ T get(const T *p) {
    if (FUSED) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return *p;
}

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

// Settle the rows of one 64-row chunk in order.  cand: the rows still clear
// whose word d (lane k holds row k's word for the chunk's own tile) is
// nonzero; rows with a zero word remove nothing inside the chunk.  The
// lowest candidate is kept and ORs its word into rem, which may remove later
// candidates; then the next.  Returns rem.
__device__ __forceinline__ uint64_t settle_rows(uint64_t d, uint64_t rem, uint64_t cand) {
    while (cand) {
        const int k = __builtin_ctzll(cand);
        rem |= read_lane64(d, k);
        cand &= cand - 1ull;  // row k settled
        cand &= ~rem;         // rows it removed
    }
    return rem;
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

constexpr int APPLIERS = NWAVES - 1;
// Bounded waits: about a second of polling before a wait gives up.
constexpr uint32_t SPIN_LIMIT = 1u << 23;

// Entries of a row tile's list held in registers: rounds of 64, in each of
// an applier's two register sets; the rest is read when the kept set is
// known.  The plain sweep's one workgroup has registers to spare and holds
// 1536 entries (217 VGPRs); the fused sweep shares its kernel's register
// budget with the mask and holds 384.  A build holding the whole 2048-entry
// list (256 VGPRs, no spills, no scratch, the resolver's code identical
// instruction for instruction) gave wrong kept sets in about 5 % of the calls
// on 8192 clustered boxes; the 1536- and 1024-entry builds gave none in 300
// calls each.  That build issued up to 71 vector loads per applier wave
// without a wait, more than the wave's vector-memory counter holds (see
// VMCNT_CAPACITY below); the sizes are kept under both limits.
template <bool FUSED>
constexpr int rmax() { return FUSED ? 6 : 24; }

// An applier issues, without a wait in between, the loads of one register
// set (two per round: word index and value) and of the next chunk's first
// level (NEAR + 1 words, the list length, the order entry).  The wave's
// vector-memory counter holds at most 63 outstanding instructions; the
// 2048-entry build that gave wrong kept sets was the only one that issued
// more (71), so the count is kept under the counter's capacity.
constexpr int VMCNT_CAPACITY = 63;
static_assert(2 * rmax<false>() + (NEAR_TILES + 1) + 2 <= VMCNT_CAPACITY &&
                  2 * rmax<true>() + (NEAR_TILES + 1) + 2 <= VMCNT_CAPACITY,
              "an applier's loads in flight must fit the vector-memory counter");

constexpr int NEAR = NEAR_TILES;
static_assert(NEAR >= 2, "the resolver carries the words for the next two tiles in registers");
// Word c is complete once chunk c - LAG and every chunk before it is applied.
constexpr int LAG = NEAR + 1;

// Appliers have slack; their polling shares the LDS with the resolver.
constexpr int APPLIER_SLEEP = 1;

// Chunk c's data sits in ring slot c mod RING.  An applier stages chunk x
// (A = APPLIERS) before it waits for chunk x - A, so the last settlement it
// has seen is that of x - 2A, its chunk before last.  The resolver reads a
// chunk's slot while settling the chunk two before it and, if the data was
// late, while settling the chunk itself; so once x - 2A is settled the slot's
// previous chunk, x - RING <= x - 2A, is read for the last time.  The settled
// word and offset the resolver leaves for chunk c are read by chunk c's
// applier before it reports chunk c applied, and the resolver reaches chunk
// c + LAG < c + RING only after that report.  (tests/test_sweep_protocol.py
// runs a model of this hand-over under random interleavings.)
constexpr int RING = 16;
static_assert(RING >= 2 * APPLIERS && RING > LAG && (RING & (RING - 1)) == 0,
              "the staging ring must outlast an applier's lead over the resolver");

struct StageSlot {
    uint64_t near[NEAR + 1][64];  // lane k: row 64c + k's words for tiles c .. c + NEAR
    uint64_t nzn;  // rows with a nonzero word for one of the next NEAR tiles
    // Both c + 1 when set, read together as one 64-bit word: ready once the
    // words above are staged, app_lag once chunk c - LAG is applied (its
    // applier writes it here, so one read tells the resolver both).
    uint32_t ready, app_lag;
};

struct Settled {
    uint64_t rem;    // settled removed word of the chunk
    uint32_t k_off;  // boxes kept before the chunk (one image)
    uint32_t pad;
};

struct SweepSmem {
    StageSlot stage[RING];
    // settled[c mod RING] is chunk c's; the resolver's lanes other than lane
    // 0 direct their copies of those writes to settled[RING + lane] and
    // resolved[lane] (every lane stores, so the stores need no branch and
    // the number of LDS accesses per chunk is fixed)
    Settled settled[RING + 64];
    uint32_t resolved[64];  // [0]: chunks settled
    uint32_t kept_total;
    uint32_t abort;
    uint32_t done_upto;  // fused kernel: row tiles below this are known finished
    uint32_t poller;     // fused kernel: 1 while a wave reads the mask's counters
};

// Hand-over flags.  Everything handed over between waves lives in LDS, and
// the LDS unit performs one wave's operations in the order they are issued.
// So a writer that issues its data writes and then the flag write, and a
// reader that sees the flag and only then issues its data reads, are ordered
// by the hardware; only the compiler must be kept from moving memory accesses
// across the flag (the empty asm with a memory clobber).  Workgroup-scope
// release/acquire would also be correct, but a release waits for every
// outstanding global load, stalling the prefetch this kernel relies on.
__device__ __forceinline__ void compiler_barrier() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t flag_load(const uint32_t *p) {
    const uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    compiler_barrier();
    return v;
}
__device__ __forceinline__ void flag_store(uint32_t *p, uint32_t v) {
    compiler_barrier();
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// sm.abort values.  ABORT_ERROR: a wait gave up (internal error raised).
// ABORT_NEEDS_DENSE: a tile's list overflowed and there are no dense rows
// (FLAG_NEEDS_DENSE raised: the call runs again with them).
// ABORT_BAIL: the fused sweep stops without a result (a tile's list
// overflowed, or the mask took too long); its post says so, and the host
// runs the plain sweep kernel on the finished mask.
constexpr uint32_t ABORT_ERROR = 1u;
constexpr uint32_t ABORT_BAIL = 2u;
constexpr uint32_t ABORT_NEEDS_DENSE = 3u;

// Give up: the fused sweep bails out quietly, the plain sweep reports an
// internal error.
template <bool FUSED>
__device__ __forceinline__ void give_up(SweepSmem &sm, Ctrl *ctrl) {
    if ((threadIdx.x & 63) == 0) {
        flag_store(&sm.abort, FUSED ? ABORT_BAIL : ABORT_ERROR);
        if (!FUSED) atomicOr(&ctrl->error, ERR_INTERNAL);
    }
}

// Wait until *flag >= target.  Returns false if it takes too long (and gives
// up) or another wave gave up.
template <bool FUSED, int SLEEP = 1>
__device__ __forceinline__ bool wait_flag(const uint32_t *flag, uint32_t target, SweepSmem &sm,
                                          Ctrl *ctrl) {
    uint32_t spins = 0;
    while (flag_load(flag) < target) {
        if (flag_load(&sm.abort)) return false;
        if (++spins > SPIN_LIMIT) {
            give_up<FUSED>(sm, ctrl);
            return false;
        }
        __builtin_amdgcn_s_sleep(SLEEP);
    }
    return true;
}

// Fused kernel: wait until every mask work item of row tile c has finished
// (each adds 64 to done[c] after its stores have completed).  Row tiles
// finish roughly in order, so the waves share a frontier in LDS (every tile
// below sm.done_upto has finished).  One wave at a time reads the counts of
// the 64 tiles from the frontier on, one per lane, and moves the frontier
// past those that finished in a row; the others watch the frontier.  (Device-
// scope reads of the counters that the mask's waves are raising slow down the
// mask waves on this wave's XCD, several times over when several waves poll.)
// Data a wave reads after learning of a finished tile from the frontier is
// visible to it as well: the mask's stores were visible device-wide before
// its count was raised.
__device__ __forceinline__ bool wait_tile_done(const SweepArgs &a, int c, SweepSmem &sm) {
    const int lane = threadIdx.x & 63;
    uint32_t spins = 0;
    for (;;) {
        const uint32_t base = flag_load(&sm.done_upto);
        if ((uint32_t)c < base) break;
        // claim the polling role (every lane asks; the LDS grants one)
        uint32_t expected = 0u;
        const bool claimed = lane == 0 && __hip_atomic_compare_exchange_strong(
                                              &sm.poller, &expected, 1u, __ATOMIC_RELAXED,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__ballot(claimed)) {
            const int t = (int)flag_load(&sm.done_upto) + lane;
            bool fin = false;
            if (t < a.words) {
                const uint32_t items =
                    (64u << a.done_shift) * (uint32_t)(a.strip_groups - t / a.strip);
                fin = __hip_atomic_load(&a.done[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                      items;
            }
            const uint64_t m = __ballot(fin);
            const uint32_t run = m == ~0ull ? 64u : (uint32_t)__builtin_ctzll(~m);
            // every lane stores the same values: no lane-divergent region
            // inside a loop whose exit the wave takes together
            if (run)
                __hip_atomic_fetch_max(&sm.done_upto, (uint32_t)(t - lane) + run, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            flag_store(&sm.poller, 0u);
            if ((uint32_t)c < (uint32_t)(t - lane) + run) break;
            if (run) continue;
        }
        if (flag_load(&sm.abort)) return false;
        if (++spins > SPIN_LIMIT) {
            give_up<true>(sm, a.ctrl);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    compiler_barrier();
    return true;
}

// s_waitcnt vmcnt(0): every vector memory load issued so far has returned.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// First-level data of a chunk: lane k's words for tiles c .. c + NEAR (rows
// 64c + k; zeros past n or outside the band) and the tile's list length.
struct Level1 {
    uint64_t near[NEAR + 1];
    uint32_t count;
};

// Returns false if the fused sweep gave up while waiting for the mask.
template <bool FUSED>
__device__ __forceinline__ bool load_level1(const SweepArgs &a, int c, Level1 &l, SweepSmem &sm) {
    if (FUSED && !wait_tile_done(a, c, sm)) return false;
    const int p = 64 * c + (int)(threadIdx.x & 63);
#pragma unroll
    for (int j = 0; j <= NEAR; ++j) l.near[j] = get<FUSED>(&a.tnear[(size_t)j * a.npad + p]);
    l.count = get<FUSED>(&a.tcount[c]);
    return true;
}

// Stage chunk c's near words and their summary masks for the resolver, then
// announce them.
__device__ __forceinline__ void stage_level1(const Level1 &l, int c, SweepSmem &sm) {
    const int lane = threadIdx.x & 63;
    StageSlot &s = sm.stage[c & (RING - 1)];
#pragma unroll
    for (int j = 0; j <= NEAR; ++j) s.near[j][lane] = l.near[j];
    uint64_t ahead = 0ull;
#pragma unroll
    for (int j = 1; j <= NEAR; ++j) ahead |= l.near[j];
    const uint64_t nzn = __ballot(ahead != 0ull);
    if (lane == 0) {
        s.nzn = nzn;
        flag_store(&s.ready, (uint32_t)c + 1u);
    }
}

// The tile's list entries, round i holding entry 64 i + lane.
template <int R>
struct Entries {
    uint32_t wk[R];
    uint64_t val[R];
    int32_t ord;  // order[64c + lane]: input index of the lane's box
};

__device__ __forceinline__ int rounds_of(uint32_t count) {
    const uint32_t held = count < (uint32_t)TILE_LIST_CAP ? count : (uint32_t)TILE_LIST_CAP;
    return (int)((held + 63u) / 64u);
}

template <bool FUSED>
__device__ __forceinline__ void load_entries(const SweepArgs &a, int c, int rounds,
                                             Entries<rmax<FUSED>()> &e) {
    const size_t base = (size_t)c * TILE_LIST_CAP + (threadIdx.x & 63);
    // written by the sort, before this launch: a plain load
    e.ord = a.order[64 * c + (threadIdx.x & 63)];
#pragma unroll
    for (int i = 0; i < rmax<FUSED>(); ++i) {
        if (i < rounds) {
            e.wk[i] = get<FUSED>(&a.tent_wk[base + 64 * i]);
            e.val[i] = get<FUSED>(&a.tent_val[base + 64 * i]);
        }
    }
}

__device__ __forceinline__ void apply_entry(uint32_t wk, uint64_t val, bool live, uint64_t kept,
                                            int c, uint64_t *removed) {
    const uint32_t k = wk & 63u, w = wk >> 6;
    if (live && ((kept >> k) & 1ull) && w > (uint32_t)(c + NEAR)) atomicOr(&removed[w], val);
}

// Apply rounds I, I+1, ... < rounds of the register-held entries.  Nested
// uniform branches (rather than a loop) keep every register index constant
// and skip the rounds that do not exist.
template <int I, int R>
__device__ __forceinline__ void apply_rounds(const Entries<R> &e, int rounds, uint32_t count,
                                             uint64_t kept, int c, uint64_t *removed) {
    if constexpr (I < R) {
        if (I < rounds) {
            const uint32_t lane = threadIdx.x & 63;
            apply_entry(e.wk[I], e.val[I], 64u * I + lane < count, kept, c, removed);
            apply_rounds<I + 1, R>(e, rounds, count, kept, c, removed);
        }
    }
}

// OR of a 64-bit value over the lanes of the wave (DPP prefix over rows of
// 16 lanes, then row broadcasts; lane 63 ends up holding the whole wave).
__device__ __forceinline__ uint32_t wave_or32(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
    const uint32_t lo = wave_or32((uint32_t)v);
    const uint32_t hi = wave_or32((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// What the resolver reads from LDS for one chunk, in two parts.  The staged
// part (lane k's words for row 64c + k, the summary mask and the ready flag)
// is read two chunks ahead.  The removed word and the flag that says it is
// complete are read one chunk ahead, which gives the appliers a chunk more
// to OR far words in.
struct StagedBatch {
    uint32_t ready;
    uint64_t nzn;
    uint64_t nw[NEAR + 1];
};
struct WordBatch {
    uint32_t app_lag;
    uint64_t rem;
};

// The LDS performs the reads in order, so data read after a flag that is
// already set is the data that flag announces.
__device__ __forceinline__ void read_staged(int x, SweepSmem &sm, StagedBatch &b) {
    const int lane = threadIdx.x & 63;
    const StageSlot &s = sm.stage[x & (RING - 1)];
    b.ready = flag_load(&s.ready);
    b.nzn = s.nzn;
#pragma unroll
    for (int j = 0; j <= NEAR; ++j) b.nw[j] = s.near[j][lane];
    compiler_barrier();
}
__device__ __forceinline__ void read_word(int x, const uint64_t *removed, SweepSmem &sm,
                                          WordBatch &b) {
    b.app_lag = flag_load(&sm.stage[x & (RING - 1)].app_lag);
    b.rem = removed[x];
    compiler_barrier();
}

// s_waitcnt lgkmcnt(0): every LDS access issued so far has completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Resolver state carried from chunk to chunk in scalar registers.
struct ResolverState {
    uint64_t carry;   // kept rows' words for tile c (chunk c - 1)
    bool dead;        // a wait gave up: the remaining chunks are skipped
    uint32_t total;   // boxes kept before chunk c
    // 0, in a register the compiler cannot see into: added to the address
    // of the kept rows' ORs into LDS, which then go out as one instruction
    // from every lane (the LDS unit combines the lanes) instead of a loop
    // over the lanes that the compiler makes of an atomic with one address
    int zero;
};

// Settle chunk c from its staged batch cur and its word batch wb, after
// issuing the reads of word c + 1 (into wb) and of chunk c + 2's staged
// batch (into ahead).
//
// Word c + 1 is read before chunk c is settled.  That is safe because chunk
// c's words for it travel in registers (carry), the words of chunks c - 1 ..
// c + 1 - NEAR for it were ORed into LDS (atomics) before the read is
// issued, and the far words of chunks up to c + 1 - LAG are in once the flag
// read with it says so: the flags of the chunks before have been checked (or
// waited for) before this read is issued.  Reading ahead keeps LDS latency, and this chunk's own LDS
// writes, off the path from one chunk to the next.
template <bool FUSED>
__device__ __forceinline__ void resolve_one(const SweepArgs &a, uint64_t *removed, SweepSmem &sm,
                                            int c, ResolverState &st, StagedBatch &cur,
                                            StagedBatch &ahead, WordBatch &wb) {
    const int lane = threadIdx.x & 63;
    const uint32_t want = (uint32_t)c + 1u;
    // s_waitcnt lgkmcnt(8): this chunk's batches are in.  Every chunk issues
    // the next word batch (2 reads), a staged batch (5 reads) and its
    // publishing writes (3), so word c was followed by chunk c - 1's staged
    // batch and writes.
    __builtin_amdgcn_s_waitcnt(0xC07F | (8 << 8));
    // (the flags are the same in every lane: tested in scalar registers, so
    // the compiler keeps the loop's branches uniform)
    const uint32_t ready = __builtin_amdgcn_readfirstlane(cur.ready);
    const uint32_t app = __builtin_amdgcn_readfirstlane(wb.app_lag);
    if (__builtin_expect((ready != want) | (app != want), 0)) {
        StageSlot &s = sm.stage[c & (RING - 1)];
        const bool ok = wait_flag<FUSED>(&s.ready, want, sm, a.ctrl) &&
                        wait_flag<FUSED>(&s.app_lag, want, sm, a.ctrl);
        if (!__builtin_amdgcn_readfirstlane((int)ok)) st.dead = true;
        read_staged(c, sm, cur);
        read_word(c, removed, sm, wb);
        wait_lds();
    }
    // rows past n are marked removed from the start; their words are zero
    uint64_t rem = uniform64(wb.rem) | st.carry;
    // Issued for every chunk, also past the last one (removed[] has NEAR >= 2
    // spare words and the staging slots are a ring), so that the number of
    // LDS accesses in flight is the same on every path through the loop.
    read_word(c + 1, removed, sm, wb);
    read_staged(c + 2, sm, ahead);

    rem = settle_rows(cur.nw[0], rem, ~rem & __ballot(cur.nw[0] != 0ull));
    const uint64_t kept = ~rem;
    uint64_t c1 = 0ull;
    if (kept & uniform64(cur.nzn)) {
        const bool mine = (kept >> lane) & 1ull;
        // a wave-wide OR only where some kept row has a nonzero word
        if (__ballot(mine && cur.nw[1] != 0ull)) c1 = wave_or64(mine ? cur.nw[1] : 0ull);
        if (mine) {
            // removed has NEAR spare words past the end for the last chunks
#pragma unroll
            for (int j = 2; j <= NEAR; ++j)
                if (cur.nw[j] != 0ull) atomicOr(&removed[c + j + st.zero], cur.nw[j]);
        }
    }
    st.carry = c1;
    Settled &out = sm.settled[lane == 0 ? (c & (RING - 1)) : RING + lane];
    out.rem = rem;
    out.k_off = st.total;
    flag_store(&sm.resolved[lane], want);
    st.total += (uint32_t)__popcll(kept);
}

// Resolver: settle the chunks in order.  A chunk in which no surviving row
// has a nonzero diagonal word, and no kept row a nonzero word for the next
// NEAR tiles (most chunks, when overlaps are sparse), costs only its flags,
// summary mask and removed word.  Otherwise the kept rows' words for tile
// c + 1 are ORed across the wave into a register, those for tiles c + 2 ..
// c + NEAR into LDS with atomics.
template <bool FUSED>
__device__ void resolve_chunks(const SweepArgs &a, uint64_t *removed, SweepSmem &sm) {
    const int W = a.words;
    ResolverState st;
    st.carry = 0ull;
    st.dead = false;
    st.total = 0u;
    asm volatile("v_mov_b32 %0, 0" : "=v"(st.zero));
    StagedBatch b0, b1, b2;
    WordBatch wb;
    read_staged(0, sm, b0);
    read_staged(1, sm, b1);
    read_word(0, removed, sm, wb);
    // Every path into the loop arrives with these batches in registers, so
    // the reads in flight inside the loop are only those issued there.
    wait_lds();
    // The first W mod 3 chunks, so that the loop settles three per trip to
    // the end: every path through its body then issues the same LDS
    // accesses, the compiler's waits stay exact and the batches keep their
    // registers from trip to trip.
    const int lead = W % 3;
    if (lead >= 1) resolve_one<FUSED>(a, removed, sm, 0, st, b0, b2, wb);
    if (lead >= 2) resolve_one<FUSED>(a, removed, sm, 1, st, b1, b0, wb);
    if (lead) {
        // read the loop's first batches afresh (each read is complete if
        // its own flag says so: every earlier flag has been checked)
        wait_lds();
        read_staged(lead, sm, b0);
        read_staged(lead + 1, sm, b1);
        read_word(lead, removed, sm, wb);
        wait_lds();
    }
    // three chunks per trip, so the three staged batches trade roles
    // without copies
    for (int c = lead; c < W; c += 3) {
        resolve_one<FUSED>(a, removed, sm, c, st, b0, b2, wb);
        resolve_one<FUSED>(a, removed, sm, c + 1, st, b1, b0, wb);
        resolve_one<FUSED>(a, removed, sm, c + 2, st, b2, b1, wb);
        // after giving up, every wait ends at once: a few chunks more are harmless
        if (st.dead) return;
    }
    if (st.dead) return;
    sm.kept_total = st.total;  // every lane stores the same value
}

// Kept rows of an overflowed tile: OR their dense words for tiles
// c + NEAR + 1 .. cend - 1, four rows and two 64-word blocks per row per round.
__device__ void apply_dense(const SweepArgs &a, int c, int stride, uint64_t kept,
                            uint64_t *removed) {
    const int lane = threadIdx.x & 63;
    const int cend = a.tile_cend[c];
    const int col0 = (c / a.strip) * a.strip;
    uint64_t rows = kept;
    while (rows) {
        int kr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            kr[t] = rows ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(rows)) : -1;
            rows &= rows - 1ull;
        }
        for (int w0 = c + NEAR + 1; w0 < cend; w0 += 128) {
            uint64_t v[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int w = w0 + 64 * j + lane;
                    v[t][j] = (kr[t] >= 0 && w < cend)
                                  ? a.mask[(size_t)(64 * c + kr[t]) * stride + (size_t)(w - col0)]
                                  : 0ull;
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (v[t][j]) atomicOr(&removed[w0 + 64 * j + lane], v[t][j]);
            }
        }
    }
}

// One chunk of an applier: chunk c's entries are in `cur`, chunk c + A's
// first level in `l1`.  Stages chunk c + A for the resolver and issues the
// loads of its entries (into `nxt`) and of chunk c + 2A's first level, all
// before waiting for chunk c's kept set, so that the memory latency of the
// next chunk overlaps the wait.  Returns false if the sweep gave up.
template <bool FUSED>
__device__ __forceinline__ bool apply_one(const SweepArgs &a, int stride, uint64_t *removed,
                                          SweepSmem &sm, int c, uint32_t &count, Level1 &l1,
                                          const Entries<rmax<FUSED>()> &cur,
                                          Entries<rmax<FUSED>()> &nxt) {
    const int lane = threadIdx.x & 63;
    const int W = a.words;
    const int A = APPLIERS;
    wait_loads();
    uint32_t count_next = 0;
    if (c + A < W) {
        stage_level1(l1, c + A, sm);
        count_next = __builtin_amdgcn_readfirstlane(l1.count);
        load_entries<FUSED>(a, c + A, rounds_of(count_next), nxt);
        if (c + 2 * A < W && !load_level1<FUSED>(a, c + 2 * A, l1, sm)) return false;
    }
    if (!wait_flag<FUSED, APPLIER_SLEEP>(&sm.resolved[0], (uint32_t)c + 1u, sm, a.ctrl))
        return false;
    // The resolver wrote the chunk's settled word and the count of boxes
    // kept before it ahead of the counter.  Both are read before the chunk
    // is reported applied: after that the resolver may reuse the slot.
    const Settled &s = sm.settled[c & (RING - 1)];
    const uint64_t kept = ~uniform64(s.rem);
    const uint32_t k_off = s.k_off;
    if (kept) {
        if (count > (uint32_t)TILE_LIST_CAP) {
            // dense rows are plain stores of the mask stage, not visible to
            // the fused sweep: leave the work to the plain sweep
            if (FUSED) {
                give_up<true>(sm, a.ctrl);
                return false;
            }
            // no dense rows this time: stop, and have the call run again
            // with them
            if (!a.dense) {
                if (lane == 0) {
                    flag_store(&sm.abort, ABORT_NEEDS_DENSE);
                    atomicOr(&a.ctrl->flags, FLAG_NEEDS_DENSE);
                }
                return false;
            }
            apply_dense(a, c, stride, kept, removed);
        } else {
            const int rounds = rounds_of(count);
            apply_rounds<0, rmax<FUSED>()>(cur, rounds, count, kept, c, removed);
            // rounds beyond the registers: load and apply them now
            const size_t base = (size_t)c * TILE_LIST_CAP + lane;
            for (int i = rmax<FUSED>(); i < rounds; ++i) {
                const uint32_t wk = get<FUSED>(&a.tent_wk[base + 64 * i]);
                const uint64_t val = get<FUSED>(&a.tent_val[base + 64 * i]);
                apply_entry(wk, val, (uint32_t)(64 * i + lane) < count, kept, c, removed);
            }
        }
    }
    if (lane == 0) flag_store(&sm.stage[(c + LAG) & (RING - 1)].app_lag, (uint32_t)(c + LAG) + 1u);
    // the outputs: off the resolver's path
    if (lane == 0) a.kept[c] = kept;
    if (!a.grouped && ((kept >> lane) & 1ull)) {
        const uint64_t below = (1ull << lane) - 1ull;
        a.keep_out[k_off + (uint32_t)__popcll(kept & below)] = (int64_t)cur.ord;
    }
    count = count_next;
    return true;
}

// Applier q (1..APPLIERS): chunks q-1, q-1+APPLIERS, ...  Loads run ahead:
// while chunk c waits for its kept set, the entries of chunk c + A and the
// first level (near words, list length) of chunk c + 2A are in flight
// (A = APPLIERS).  Two register sets of entries alternate between chunks.
template <bool FUSED>
__device__ void apply_chunks(const SweepArgs &a, int stride, uint64_t *removed, SweepSmem &sm,
                             int q) {
    const int W = a.words;
    const int A = APPLIERS;
    int c = q - 1;
    if (c >= W) return;
    Level1 l1;
    Entries<rmax<FUSED>()> ea, eb;
    // prologue: chunk c staged, its entries and chunk c + A's first level issued
    if (!load_level1<FUSED>(a, c, l1, sm)) return;
    wait_loads();
    stage_level1(l1, c, sm);
    uint32_t count = __builtin_amdgcn_readfirstlane(l1.count);
    load_entries<FUSED>(a, c, rounds_of(count), ea);
    if (c + A < W && !load_level1<FUSED>(a, c + A, l1, sm)) return;
    for (; c < W; c += 2 * A) {
        if (!apply_one<FUSED>(a, stride, removed, sm, c, count, l1, ea, eb)) return;
        if (c + A >= W) return;
        if (!apply_one<FUSED>(a, stride, removed, sm, c + A, count, l1, eb, ea)) return;
    }
}

// The whole sweep in one workgroup: LDS set-up, the resolver and applier
// waves, then the kept bitmap and (one image) the compaction.
template <bool FUSED>
__device__ __forceinline__ void sweep_body(const SweepArgs &a, uint64_t *removed, SweepSmem &sm) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int W = a.words, n = a.n;
    const int stride = a.grouped ? a.ctrl->band_stride : a.mstride;

    // rows past n start out removed, so no chunk ever keeps them
    for (int w = tid; w < W + NEAR_TILES; w += NT) removed[w] = w == W - 1 ? ~rows_valid(w, n) : 0ull;
    if (tid < RING) {
        sm.stage[tid].ready = 0u;
        // chunks below LAG wait for no earlier chunk
        sm.stage[tid].app_lag = tid < LAG ? (uint32_t)tid + 1u : 0u;
    }
    if (tid == 0) {
        sm.resolved[0] = 0u;
        sm.abort = 0u;
        sm.done_upto = 0u;
        sm.poller = 0u;
    }
    __syncthreads();

    const int wv = __builtin_amdgcn_readfirstlane(wave);
    if (wv == 0) resolve_chunks<FUSED>(a, removed, sm);
    else apply_chunks<FUSED>(a, stride, removed, sm, wv);
    __syncthreads();
    if (sm.abort) return;

    // the appliers wrote the kept bitmap
    if (a.grouped) return;
    // one image: the appliers have written the output
    if (tid == 0) {
        a.ctrl->count = (int32_t)sm.kept_total;
        if (FUSED) a.ctrl->sweep_done = 1u;
    }
}

// Waves of a workgroup that posts the call's result: every wave's stores
// complete (s_waitcnt vmcnt(0)), then one thread posts.
__device__ __forceinline__ void post_from_workgroup(const Post &p, const Ctrl *ctrl, bool valid) {
    if (p.dst == nullptr) return;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (threadIdx.x == 0) post_result(p, ctrl, valid);
}

__global__ __launch_bounds__(NT) void sweep_kernel(SweepArgs a) {
    extern __shared__ uint64_t removed[];
    __shared__ SweepSmem sm;
    // the grouped sweep (which runs whenever every band fits its window)
    // may already have produced the result; after a fused launch this
    // kernel runs only when that sweep stopped, and finds sweep_done clear
    const bool done = a.ctrl->sweep_done ||
                      (a.grouped && a.ctrl->band_stride <= GROUP_SWEEP_WIN);
    if (!done) sweep_body<false>(a, removed, sm);
    post_from_workgroup(a.post, a.ctrl, true);
}

// ---------------------------------------------------------------- grouped sweep

constexpr int GS_THREADS = 256;
constexpr int GS_WAVES = GS_THREADS / 64;

struct GroupSweepArgs {
    const uint64_t *mask;
    const int32_t *seg_start;
    const Ctrl *ctrl;
    uint64_t *kept;
    int n, strip;
};

// Grouped input: boxes of different (image, class) groups never suppress
// each other -- their bits in each other's words are zero -- so every group
// (segment of sorted positions) can be swept on its own.  One wave per
// segment walks the segment's row tiles in order: the diagonal words settle
// the segment's rows of the tile as in the plain resolver, then the kept
// rows' words for the later tiles of the segment are ORed across the wave
// into a ring of removed words kept in LDS, one slot per row tile ahead.
// Segments sharing a row tile OR their kept rows into its kept word.
__global__ __launch_bounds__(GS_THREADS) void group_sweep_kernel(GroupSweepArgs a) {
    __shared__ uint64_t ring[GS_WAVES][GROUP_SWEEP_WIN];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int stride = a.ctrl->band_stride;
    if (stride > GROUP_SWEEP_WIN) return;  // the plain sweep does the work
    const int nseg = a.ctrl->num_segments;
    const int S = a.strip;
    uint64_t *rw = ring[wave];
    for (int j = lane; j < GROUP_SWEEP_WIN; j += 64) rw[j] = 0ull;
    for (int g = blockIdx.x * GS_WAVES + wave; g < nseg; g += gridDim.x * GS_WAVES) {
        const int s0 = a.seg_start[g], s1 = a.seg_start[g + 1];
        const int t0 = s0 >> 6, tl = (s1 - 1) >> 6;
        for (int t = t0; t <= tl; ++t) {
            const int p = 64 * t + lane;
            const bool in_seg = p >= s0 && p < s1;
            // word c of row p sits at row[c]: rows hold their band only, and
            // the band of any row of the segment reaches the segment's end
            const uint64_t *row = a.mask + (size_t)p * stride - (t / S) * S;
            const uint64_t d = in_seg ? row[t] : 0ull;
            uint64_t rem = uniform64(rw[t % GROUP_SWEEP_WIN]);
            const uint64_t valid = __ballot(in_seg);
            rem = settle_rows(d, rem, ~rem & __ballot(d != 0ull) & valid);
            const uint64_t kept = ~rem & valid;
            const bool mine = (kept >> lane) & 1ull;
            for (int u = t + 1; u <= tl; ++u) {
                const uint64_t wu = mine ? row[u] : 0ull;
                if (__ballot(wu != 0ull)) {
                    const uint64_t o = wave_or64(wu);
                    if (lane == 0) rw[u % GROUP_SWEEP_WIN] |= o;
                }
            }
            if (lane == 0) {
                rw[t % GROUP_SWEEP_WIN] = 0ull;  // free for row tile t + GROUP_SWEEP_WIN
                if (kept) atomicOr(&a.kept[t], kept);
            }
        }
    }
}

// Mask work items per workgroup of the fused launch: four per wave, taken
// from the block's queue in LDS.
constexpr int FUSED_BLOCK_ITEMS = 4 * NWAVES;
// Workgroups go to the XCDs in turn (workgroup b to XCD b mod 8), and the
// XCD that holds the sweep's workgroup computes its share of the mask more
// slowly (measured: its last item ended 25 us after the others' at 65,536
// boxes, about 7 %), so its workgroups take fewer items.
constexpr int FUSED_XCDS = 8;
constexpr int FUSED_BLOCK_ITEMS_SWEEP_XCD = FUSED_BLOCK_ITEMS - 2;

// First item of mask workgroup b (b >= 1; workgroup 0 is the sweep).
__host__ __device__ __forceinline__ int64_t fused_block_start(int64_t b) {
    const int64_t before = b - 1, on_sweep_xcd = before / FUSED_XCDS;
    return (before - on_sweep_xcd) * FUSED_BLOCK_ITEMS +
           on_sweep_xcd * FUSED_BLOCK_ITEMS_SWEEP_XCD;
}

// Mask and sweep in one launch (one image).  Workgroup 0 runs the sweep;
// each of the other workgroups computes a block of FUSED_BLOCK_ITEMS mask
// work items, its waves taking the block's items one at a time from a
// counter in LDS.  The GPU starts workgroups in order as earlier ones
// leave, so items start row tile by row tile, and a wave that finishes an
// item early takes the next one rather than idling until its workgroup's
// slowest wave is done.
// The sweep follows the finished row tiles while later ones are still being
// computed.  No mask wave ever waits for anything, so every item completes
// whatever the order in which workgroups are scheduled.
// (two workgroups per compute unit, 4 waves per SIMD: at most 128 registers)
__global__ __launch_bounds__(NT, 6) void mask_sweep_kernel(
    maskcore::MaskArgs ma, const Ctrl *ctrl, const float4 *__restrict__ sb,
    const float *__restrict__ area, const int32_t *__restrict__ tile_cend,
    const int32_t *__restrict__ item_base, uint64_t *__restrict__ mask,
    uint32_t *__restrict__ tcount, uint32_t *__restrict__ tent_wk,
    uint64_t *__restrict__ tent_val, uint64_t *__restrict__ tnear, uint32_t *__restrict__ done,
    const uint32_t *__restrict__ scol, SweepArgs sa) {
    extern __shared__ uint64_t removed[];
    __shared__ SweepSmem sm;
    if (blockIdx.x == 0) {
        // the sweep's workgroup posts the call's result (sweep_done clear if
        // it stopped without one); every row it read was finished by then
        sweep_body<true>(sa, removed, sm);
        post_from_workgroup(sa.post, sa.ctrl, true);
        return;
    }
    const maskcore::MaskPtrs m_{sb,     area,   nullptr, tile_cend, item_base,
                                mask,   tcount, tent_wk, tent_val,  tnear,     scol};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ uint32_t item_queue;
    if (threadIdx.x == 0) item_queue = 0u;
    __syncthreads();
    (void)wave;
    maskcore::mask_items<STRIP_SINGLE, false, true, true>(
        ma, m_, ctrl, (int)fused_block_start(blockIdx.x),
        (int)(fused_block_start(blockIdx.x + 1) - fused_block_start(blockIdx.x)), done,
        &item_queue);
}

// ---------------------------------------------------------------- small inputs

// One image of at most SMALL_MAX boxes in one launch: sort, mask, sweep and
// output, so that a call costs one launch and the read-back (the page's
// measured losses at 1024 and 2048 boxes come from fixed per-launch costs:
// "LeetCUDA 14-nms", measured results).  Workgroups, in launch order:
//   0 .. W - 1   rank the 64 boxes of chunk k (the ranking sort's code);
//   W            checks the input and writes the control block;
//   W + 1        the sweep, as in the fused launch;
//   W + 2 ...    the mask, one work item per wave.
// The first W + 1 share the per-call initialisation and never wait; each
// then stores the call's epoch in its slot of `arrive`.  Every later
// workgroup first waits until all W + 1 slots hold the epoch.  The GPU starts
// workgroups in launch order, so a waiting workgroup waits only for ones
// already started, which finish whatever else is resident; the sweep also
// waits for mask items, which never wait for the sweep.  Every wait is
// bounded: a wait that gives up leaves sweep_done clear, and so does a row
// tile whose list overflowed (its dense rows are plain stores), and the host
// then runs the multi-launch path from the start.
//
// The host gives every call a new 64-bit epoch (a process-wide counter from a
// random start), so a slot left by an earlier call, or never written, does
// not match; a match of all W + 1 slots by leftover memory is not a practical
// concern.
constexpr int SMALL_PER_THREAD = SMALL_MAX / NT;  // inputs each checking thread reads
static_assert(SMALL_PER_THREAD * NT == SMALL_MAX && SMALL_MAX <= RANK_SORT_MAX,
              "small-input tiling");
static_assert(SMALL_MAX / 64 + 1 <= 128, "a wave polls at most two slots per lane");

struct SmallArgs {
    KeysArgs ka;
    const float4 *boxes;
    uint64_t *arrive;  // W + 1 slots
    uint64_t epoch;
    int prep;          // W + 1 preparing workgroups
    int mask_waves;    // waves of the mask workgroups
    Post post;         // posted by the sweep's workgroup
};

// Preparing workgroup: once every wave's device-scope stores have completed
// (s_waitcnt vmcnt(0): they reached the memory all XCDs share), one store
// of the epoch announces them.  (A release fence would also write back this
// XCD's whole L2, which cost several microseconds per workgroup here.)
__device__ __forceinline__ void announce(uint64_t *slot, uint64_t epoch) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(slot, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every preparing workgroup has announced its stores: wave 0
// polls the slots (lane l reads slots l, l + 64); false if it took too long.
__device__ __forceinline__ bool wait_prepared(const SmallArgs &s, uint32_t *ok_sh) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        uint32_t spins = 0;
        bool ok = true;
        for (;;) {
            // both loads in flight together
            const uint64_t v0 = lane < s.prep ? __hip_atomic_load(&s.arrive[lane], __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_AGENT)
                                              : s.epoch;
            const uint64_t v1 = lane + 64 < s.prep
                                    ? __hip_atomic_load(&s.arrive[lane + 64], __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : s.epoch;
            if (__ballot(v0 != s.epoch || v1 != s.epoch) == 0ull) break;
            if (++spins > SPIN_LIMIT) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane == 0) *ok_sh = ok ? 1u : 0u;
    }
    // No cache invalidation is needed after the wait: every cache was
    // invalidated when the launch began, nothing reads the prepared data
    // before this point, and the preparing workgroups' device-scope stores
    // are in memory, so the first reads of those lines fetch the new values.
    __syncthreads();
    return *ok_sh != 0u;
}

// (at most 128 registers: the sweep's and the mask's code paths share them)
__global__ __launch_bounds__(NT, 4) void small_nms_kernel(SmallArgs s, maskcore::MaskArgs ma,
                                                          SweepArgs sa) {
    extern __shared__ uint64_t removed[];
    // the sweep's shared state, or a ranking workgroup's staged scores
    __shared__ union {
        SweepSmem sweep;
        float scores[SMALL_MAX];
    } u;
    __shared__ uint32_t part[NWAVES][64];
    __shared__ uint32_t err_sh, unordered_sh, ok_sh;
    const int b = blockIdx.x;
    if (b < s.prep) {
        // the initialisation stores come last: a wait for a load (or for a
        // register a load still writes) waits for every store issued
        // before it, and device-scope stores take a round trip to memory
        if (b == s.prep - 1) {
            check_image<NT, SMALL_PER_THREAD, true>(s.ka, s.boxes, &err_sh, &unordered_sh);
        } else {
            RankStaged<NWAVES, SMALL_MAX> st;
            rank_staged_load(s.ka, s.boxes, b, st);
            rank_staged_finish(s.ka, s.boxes, b, st, u.scores, part);
        }
        per_call_init<false, true>(s.ka, b * NT + threadIdx.x, s.prep * NT);
        announce(&s.arrive[b], s.epoch);
        return;
    }
    const bool ready = wait_prepared(s, &ok_sh);
    if (b == s.prep) {
        // the sweep posts the call's result, or "no result" if the wait gave
        // up (the control block may then be incomplete)
        if (ready) sweep_body<true>(sa, removed, u.sweep);
        post_from_workgroup(s.post, sa.ctrl, ready);
        return;
    }
    if (!ready) return;
    const Work &w = s.ka.w;
    const maskcore::MaskPtrs m_{w.sb,     w.area,   nullptr,    w.tile_cend, w.item_base, w.mask,
                                w.tcount, w.tent_wk, w.tent_val, w.tnear,     w.scol};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    maskcore::mask_items<STRIP_SINGLE, false, true, false, true>(
        ma, m_, w.ctrl, (b - s.prep - 1) * NWAVES + wave, s.mask_waves, w.done);
}

// The call's result, posted after the last kernel where that kernel has
// many workgroups (stream order makes it wait for all of them).
__global__ __launch_bounds__(64) void publish_kernel(Post p, const Ctrl *ctrl) {
    if (threadIdx.x == 0) post_result(p, ctrl, true);
}

// ---------------------------------------------------------------- compaction

struct CompactArgs {
    const int32_t *score_order;
    const int32_t *inv;
    const uint64_t *kept;
    uint32_t *block_cnt;
    Ctrl *ctrl;
    int64_t *keep_out;
    int n, blocks;
};

constexpr int CT = 256;  // compaction threads per workgroup
constexpr int CT_ROWS = COMPACT_CHUNK / CT;

// Score rank r's input index and whether it was kept (its sorted position's
// bit in the kept bitmap).
// Both lookups are clamped into [0, n): a call whose sort gave up (an
// error, or a sort to be run again) may leave stale entries, and its result
// is discarded, but no read may leave the arrays.
__device__ __forceinline__ bool rank_kept(const CompactArgs &a, int r, int32_t &i) {
    i = min((uint32_t)a.score_order[r], (uint32_t)(a.n - 1));
    const int p = (int)min((uint32_t)a.inv[i], (uint32_t)(a.n - 1));
    return (a.kept[p >> 6] >> (p & 63)) & 1ull;
}

// Grouped input, pass 1: kept boxes per block of COMPACT_CHUNK score ranks.
__global__ __launch_bounds__(CT) void compact_count_kernel(CompactArgs a) {
    __shared__ uint32_t part[CT / 64];
    const int tid = threadIdx.x;
    const int base = blockIdx.x * COMPACT_CHUNK;
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < CT_ROWS; ++j) {
        const int r = base + j * CT + tid;
        int32_t i;
        if (r < a.n && rank_kept(a, r, i)) ++cnt;
    }
    cnt = wave_incl_sum(cnt);
    if ((tid & 63) == 63) part[tid >> 6] = cnt;
    __syncthreads();
    if (tid == 0) {
        uint32_t t = 0;
        for (int q = 0; q < CT / 64; ++q) t += part[q];
        a.block_cnt[blockIdx.x] = t;
    }
}

// Grouped input, pass 2: each block writes its kept input indices in score
// order, after the kept boxes of all earlier blocks; the last block stores
// the count.
__global__ __launch_bounds__(CT) void compact_write_kernel(CompactArgs a) {
    __shared__ uint32_t part[CT / 64];
    __shared__ uint32_t base_sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t before = 0;
    for (int b = tid; b < (int)blockIdx.x; b += CT) before += a.block_cnt[b];
    before = wave_incl_sum(before);
    if (lane == 63) part[wave] = before;
    __syncthreads();
    if (tid == 0) {
        uint32_t t = 0;
        for (int q = 0; q < CT / 64; ++q) t += part[q];
        base_sh = t;
    }
    __syncthreads();
    uint32_t pos = base_sh;
    const int base = blockIdx.x * COMPACT_CHUNK;
    for (int j = 0; j < CT_ROWS; ++j) {
        const int r = base + j * CT + tid;
        int32_t i = 0;
        const bool k = r < a.n && rank_kept(a, r, i);
        // ranks of this row in thread order: wave counts, then lanes
        const uint64_t m = __ballot(k);
        __syncthreads();
        if (lane == 0) part[wave] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t off = 0, row_total = 0;
        for (int q = 0; q < CT / 64; ++q) {
            if (q < wave) off += part[q];
            row_total += part[q];
        }
        const uint32_t in_wave =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (k) a.keep_out[pos + off + in_wave] = (int64_t)i;
        pos += row_total;
    }
    if (blockIdx.x == (unsigned)(a.blocks - 1) && tid == 0) a.ctrl->count = (int32_t)pos;
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

SweepArgs make_sweep_args(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out) {
    SweepArgs a;
    a.mask = w.mask;
    a.tile_cend = w.tile_cend;
    a.order = w.order;
    a.tcount = w.tcount;
    a.tent_wk = w.tent_wk;
    a.tent_val = w.tent_val;
    a.tnear = w.tnear;
    a.ctrl = w.ctrl;
    a.kept = w.kept;
    a.keep_out = keep_out;
    a.n = P.n;
    a.words = (int)L.words;
    a.npad = (int)L.npad;
    a.mstride = (int)L.mstride;
    a.strip = P.strip;
    a.grouped = P.grouped ? 1 : 0;
    a.done = w.done;
    a.strip_groups = (int)((L.words + P.strip - 1) / P.strip);
    a.done_shift = 0;
    a.dense = P.dense ? 1 : 0;
    a.post = Post{nullptr, 0};
    return a;
}

}  // namespace

hipError_t launch_sweep(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                        hipStream_t stream, const Post &post) {
    SweepArgs a = make_sweep_args(P, L, w, keep_out);
    a.post = post;
    const size_t lds = (size_t)(L.words + NEAR_TILES) * sizeof(uint64_t);
    hipLaunchKernelGGL(sweep_kernel, dim3(1), dim3(NT), lds, stream, a);
    return hipGetLastError();
}

// Workgroups of the fused kernel resident per CU for a given dynamic LDS
// size (asked once per device and KiB of LDS: the query costs more than a
// launch).  The registers allow three; a large removed bitmap leaves LDS for
// two.
int fused_blocks_per_cu(size_t lds) {
    constexpr int BUCKETS = (FUSE_MAX_WORDS + NEAR_TILES) * 8 / 1024 + 1;
    static int cached[64][BUCKETS] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int b = (int)((lds + 1023) / 1024);
    if (b >= BUCKETS) b = BUCKETS - 1;
    if (cached[dev][b] == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mask_sweep_kernel, NT,
                                                         (size_t)b * 1024) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        cached[dev][b] = per_cu;
    }
    return cached[dev][b];
}

// one work item per mask wave; the number of resident waves only sets how
// finely the pairs are split
static maskcore::MaskArgs fused_mask_args(const Problem &P, const Layout &L) {
    const size_t lds = (size_t)(L.words + NEAR_TILES) * sizeof(uint64_t);
    const int per_cu = fused_blocks_per_cu(lds);
    const int64_t cap = (int64_t)device_cu_count() * per_cu - 1;
    return maskcore::make_mask_args(P, L, (cap > 1 ? cap : 1) * NWAVES);
}

int fused_mask_qshift(const Problem &P, const Layout &L) { return fused_mask_args(P, L).qshift; }

bool fused_launch_applies(const Problem &P, const Layout &L) {
    if (P.grouped || L.words < FUSE_MIN_WORDS || L.words > FUSE_MAX_WORDS) return false;
    // the fused kernel holds only the pre-test form of the division-free test
    const maskcore::MaskArgs ma = fused_mask_args(P, L);
    return ma.use_packs && ma.qshift == 0;
}

hipError_t launch_mask_sweep(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                             hipStream_t stream, const Post &post) {
    if (!fused_launch_applies(P, L)) return hipErrorInvalidValue;
    const SweepArgs sa = make_sweep_args(P, L, w, keep_out);
    const size_t lds = (size_t)(L.words + NEAR_TILES) * sizeof(uint64_t);
    const maskcore::MaskArgs ma = fused_mask_args(P, L);
    const int64_t pairs = maskcore::mask_items_upper_bound(P, L);
    const int64_t items = pairs << ma.qshift;
    // one block of items per mask workgroup (fewer on the sweep's XCD)
    int64_t blocks = (items + FUSED_BLOCK_ITEMS - 1) / FUSED_BLOCK_ITEMS;
    while (fused_block_start(blocks + 1) < items) ++blocks;
    // (the grid's thread count must fit in 32 bits)
    if (blocks > MAX_GRID_THREADS / NT - 1) return hipErrorInvalidValue;
    if (blocks < 1) blocks = 1;
    SweepArgs sa2 = sa;
    sa2.done_shift = ma.qshift;  // a finished pair counts 64 << qshift
    sa2.post = post;
    hipLaunchKernelGGL(mask_sweep_kernel, dim3((unsigned)(blocks + 1)), dim3(NT), lds, stream, ma,
                       w.ctrl, w.sb, w.area, w.tile_cend, w.item_base, w.mask, w.tcount,
                       w.tent_wk, w.tent_val, w.tnear, w.done, w.scol, sa2);
    return hipGetLastError();
}

hipError_t launch_publish(const Work &w, const Post &post, hipStream_t stream) {
    if (post.dst == nullptr) return hipSuccess;
    hipLaunchKernelGGL(publish_kernel, dim3(1), dim3(64), 0, stream, post, (const Ctrl *)w.ctrl);
    return hipGetLastError();
}

bool small_launch_applies(const Problem &P) {
    return !P.grouped && P.n >= 1 && P.n <= SMALL_MAX;
}

hipError_t launch_small(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                        uint64_t epoch, const Post &post, hipStream_t stream) {
    if (!small_launch_applies(P)) return hipErrorInvalidValue;
    SmallArgs s;
    KeysArgs &ka = s.ka;
    ka.boxes = reinterpret_cast<const float4 *>(P.boxes);
    ka.scores = P.scores;
    ka.class_ids = nullptr;
    ka.offsets = nullptr;
    ka.num_images = 1;
    ka.n = P.n;
    ka.npad = (int)L.npad;
    ka.words = (int)L.words;
    ka.strip = P.strip;
    ka.mstride = (int)L.mstride;
    ka.tiles = (int)L.tiles;
    ka.grouped = 0;
    ka.w = w;
    s.boxes = ka.boxes;
    s.arrive = w.arrive;
    s.epoch = epoch;
    s.prep = (int)L.words + 1;
    s.post = post;
    // one work item per wave; the pairs are split into row groups while the
    // items fit 16 waves per CU
    maskcore::MaskArgs ma = maskcore::make_mask_args(P, L, (int64_t)device_cu_count() * 16);
    // every row tile covers all column tiles: the item count is known here
    ma.items_known = (int)maskcore::mask_items_upper_bound(P, L);
    const int64_t items = (int64_t)ma.items_known << ma.qshift;
    const int64_t mask_blocks = (items + NWAVES - 1) / NWAVES;
    s.mask_waves = (int)(mask_blocks * NWAVES);
    SweepArgs sa = make_sweep_args(P, L, w, keep_out);
    sa.done_shift = ma.qshift;  // a finished pair counts 64 << qshift
    const size_t lds = (size_t)(L.words + NEAR_TILES) * sizeof(uint64_t);
    hipLaunchKernelGGL(small_nms_kernel, dim3((unsigned)(s.prep + 1 + mask_blocks)), dim3(NT),
                       lds, stream, s, ma, sa);
    return hipGetLastError();
}

hipError_t launch_compact(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                          hipStream_t stream) {
    (void)L;
    CompactArgs a;
    a.score_order = w.score_order;
    a.inv = w.inv;
    a.kept = w.kept;
    a.block_cnt = w.block_cnt;
    a.ctrl = w.ctrl;
    a.keep_out = keep_out;
    a.n = P.n;
    a.blocks = (P.n + COMPACT_CHUNK - 1) / COMPACT_CHUNK;
    hipLaunchKernelGGL(compact_count_kernel, dim3(a.blocks), dim3(CT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(compact_write_kernel, dim3(a.blocks), dim3(CT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_group_sweep(const Problem &P, const Layout &L, const Work &w,
                              hipStream_t stream) {
    GroupSweepArgs a;
    a.mask = w.mask;
    a.seg_start = w.seg_start;
    a.ctrl = w.ctrl;
    a.kept = w.kept;
    a.n = P.n;
    a.strip = P.strip;
    // one wave per segment, segments are at most n
    int64_t blocks = (P.n + GS_WAVES - 1) / GS_WAVES;
    const int64_t cap = (int64_t)device_cu_count() * 4;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(group_sweep_kernel, dim3((unsigned)blocks), dim3(GS_THREADS), 0, stream, a);
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
