// Host side of libgreedy_nms: argument checks, workspace carve-up, stage
// launches on the caller's stream, and the end of every call: the result
// {error bits, flags, kept count} that the last kernel posts into pinned
// host memory (or, without a pinned buffer, one device-to-host copy and a
// stream synchronisation).
#include <hip/hip_runtime.h>

#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cstddef>
#include <cmath>
#include <cstring>

#include "greedy_nms.h"
#include "nms_internal.h"

namespace gnms {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool make_layout(int64_t n, Layout *out) {
    Layout L;
    L.n = n;
    L.words = (n + 63) / 64;
    L.npad = 64 * L.words;
    // worst-case row stride over both strip widths (a multiple of 16 words)
    L.mstride = ((L.words + STRIP_SINGLE - 1) / STRIP_SINGLE) * STRIP_SINGLE;
    L.tiles = (L.npad + RADIX_TILE - 1) / RADIX_TILE;
    const size_t np = (size_t)L.npad;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    L.off_ctrl = take(sizeof(Ctrl));
    L.off_keys0 = take(np * 4);
    L.off_keys1 = take(np * 4);
    L.off_vals0 = take(np * 4);
    L.off_vals1 = take(np * 4);
    L.off_order = take(np * 4);
    L.off_score_order = take(np * 4);
    L.off_seg = take(np * 4);
    L.off_inv = take(np * 4);
    L.off_sb = take(np * 16);
    L.off_area = take(np * 4);
    L.off_tile_cend = take((size_t)L.words * 4 + 4);
    L.off_item_base = take((size_t)L.words * 4 + 4);
    L.off_kept = take((size_t)L.words * 8 + 8);
    L.off_tcount = take((size_t)L.words * 4);
    L.off_tent_wk = take((size_t)L.words * TILE_LIST_CAP * 4);
    L.off_tent_val = take((size_t)L.words * TILE_LIST_CAP * 8);
    L.off_tnear = take(np * 8 * (NEAR_TILES + 1));
    L.off_hist_tile = take((size_t)L.tiles * RADIX_PASSES * 256 * 4);
    L.off_lb_status = take((size_t)RADIX_PASSES * L.tiles * 256 * 4);
    L.off_err_tile = take((size_t)L.tiles * 4);
    L.off_gcls = take(np * 4);
    L.off_gimg = take(np * 4);
    L.off_pass_plan = take(RADIX_PASSES * sizeof(RadixPassPlan));
    L.off_gbase = take((size_t)RADIX_PASSES * 256 * 4);
    L.off_done = take((size_t)L.words * 4);
    L.off_seg_start = take(np * 4 + 4);
    L.off_start_bits = take((size_t)L.words * 8);
    L.off_block_cnt = take(((size_t)n / COMPACT_CHUNK + 1) * 4);
    L.off_momax = take(np * 4);
    L.off_mscore = take(np * 4);
    L.off_mlo = take(np * 8);
    L.off_mhi = take(np * 8);
    L.off_mdrop = take((size_t)L.words * 8 + 8);
    L.off_tile_ext = take((size_t)L.tiles * 16);
    L.off_coarse = take(np * 8);  // coarse column words, then row words
    L.off_arrive = take((size_t)(L.words + 1) * 8);
    L.off_team = n <= TEAM_MAX_N ? take(team_ws_bytes(team_layout_members(n))) : 0;
    L.off_team_ring = n <= TEAM_MAX_N ? take((size_t)3 * 2 * 8 * np) : 0;
    L.off_mask = take((size_t)n * (size_t)L.mstride * 8);
    L.total = off;
    *out = L;
    return true;
}

Work carve(void *workspace, const Layout &L) {
    char *b = static_cast<char *>(workspace);
    Work w;
    w.ctrl = reinterpret_cast<Ctrl *>(b + L.off_ctrl);
    w.keys0 = reinterpret_cast<uint32_t *>(b + L.off_keys0);
    w.keys1 = reinterpret_cast<uint32_t *>(b + L.off_keys1);
    w.vals0 = reinterpret_cast<uint32_t *>(b + L.off_vals0);
    w.vals1 = reinterpret_cast<uint32_t *>(b + L.off_vals1);
    w.order = reinterpret_cast<int32_t *>(b + L.off_order);
    w.score_order = reinterpret_cast<int32_t *>(b + L.off_score_order);
    w.seg = reinterpret_cast<uint32_t *>(b + L.off_seg);
    w.inv = reinterpret_cast<int32_t *>(b + L.off_inv);
    w.sb = reinterpret_cast<float4 *>(b + L.off_sb);
    w.area = reinterpret_cast<float *>(b + L.off_area);
    w.tile_cend = reinterpret_cast<int32_t *>(b + L.off_tile_cend);
    w.item_base = reinterpret_cast<int32_t *>(b + L.off_item_base);
    w.kept = reinterpret_cast<uint64_t *>(b + L.off_kept);
    w.tcount = reinterpret_cast<uint32_t *>(b + L.off_tcount);
    w.tent_wk = reinterpret_cast<uint32_t *>(b + L.off_tent_wk);
    w.tent_val = reinterpret_cast<uint64_t *>(b + L.off_tent_val);
    w.tnear = reinterpret_cast<uint64_t *>(b + L.off_tnear);
    w.hist_tile = reinterpret_cast<uint32_t *>(b + L.off_hist_tile);
    w.lb_status = reinterpret_cast<uint32_t *>(b + L.off_lb_status);
    w.err_tile = reinterpret_cast<uint32_t *>(b + L.off_err_tile);
    w.mask = reinterpret_cast<uint64_t *>(b + L.off_mask);
    w.done = reinterpret_cast<uint32_t *>(b + L.off_done);
    w.seg_start = reinterpret_cast<int32_t *>(b + L.off_seg_start);
    w.start_bits = reinterpret_cast<uint64_t *>(b + L.off_start_bits);
    w.block_cnt = reinterpret_cast<uint32_t *>(b + L.off_block_cnt);
    w.gcls = reinterpret_cast<uint32_t *>(b + L.off_gcls);
    w.gimg = reinterpret_cast<uint32_t *>(b + L.off_gimg);
    w.pass_plan = reinterpret_cast<RadixPassPlan *>(b + L.off_pass_plan);
    w.gbase = reinterpret_cast<uint32_t *>(b + L.off_gbase);
    w.momax = reinterpret_cast<uint32_t *>(b + L.off_momax);
    w.mscore = reinterpret_cast<float *>(b + L.off_mscore);
    w.mlo = reinterpret_cast<double *>(b + L.off_mlo);
    w.mhi = reinterpret_cast<double *>(b + L.off_mhi);
    w.mdrop = reinterpret_cast<uint64_t *>(b + L.off_mdrop);
    w.tile_ext = reinterpret_cast<float4 *>(b + L.off_tile_ext);
    w.scol = reinterpret_cast<uint32_t *>(b + L.off_coarse);
    w.srow = w.scol + L.npad;
    w.arrive = reinterpret_cast<uint64_t *>(b + L.off_arrive);
    w.team = L.off_team ? reinterpret_cast<uint64_t *>(b + L.off_team) : nullptr;
    w.team_ring = L.off_team_ring ? reinterpret_cast<uint64_t *>(b + L.off_team_ring) : nullptr;
    return w;
}

namespace {

static_assert(sizeof(Readback) <= sizeof(Ctrl) && offsetof(Readback, sweep_done) ==
                                                   offsetof(Ctrl, sweep_done),
              "a copy of the control block's head fills the read-back");

// Epochs of the one-launch path for small inputs: a process-wide counter
// from a random start (clock and process id through the splitmix64
// finaliser), so that neither an earlier call's slots, of this process or
// another, nor leftover memory pass for this call's.  A function-local
// static of a trivially destructible type: nothing runs at exit.
uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t next_epoch() {
    static std::atomic<uint64_t> counter{mix64(
        (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
        ((uint64_t)getpid() << 40))};
    return counter.fetch_add(1, std::memory_order_relaxed);
}

nms_status check_common(int64_t n, float thresh, const int64_t *offsets, int64_t num_images) {
    if (n < 0 || std::isnan(thresh)) return NMS_INVALID_ARG;
    if (offsets == nullptr && num_images > 1) return NMS_INVALID_ARG;
    if (offsets != nullptr && num_images < 1) return NMS_INVALID_ARG;
    if (num_images < 0 || num_images > (int64_t)0x7fffffff) return NMS_INVALID_ARG;
    if (n > NMS_MAX_BOXES) return NMS_TOO_LARGE;
    return NMS_OK;
}

Problem make_problem(const float *boxes, const float *scores, int64_t n, float thresh,
                     const int32_t *class_ids, const int64_t *offsets, int64_t num_images) {
    Problem P;
    P.boxes = boxes;
    P.scores = scores;
    P.n = (int)n;
    P.thresh = thresh;
    P.class_ids = class_ids;
    P.offsets = offsets;
    P.num_images = offsets ? (int)num_images : 1;
    P.grouped = class_ids != nullptr || offsets != nullptr;
    P.strip = P.grouped ? STRIP_GROUPED : STRIP_SINGLE;
    P.dense = P.grouped;
    P.team_sort = true;
    P.sample_sort = false;
    return P;
}

nms_status hip_status(hipError_t e) { return e == hipSuccess ? NMS_OK : NMS_HIP_ERROR; }

// Pinned host buffers for the read-back.  A copy into pageable memory goes
// through the runtime's staging and costs tens of microseconds more per
// call.  Calls take a buffer from this pool and give it back; a buffer is
// allocated (hipHostMalloc) only when every existing one is in use, at most
// READBACK_POOL of them, and they are kept until the process ends (freeing
// them at exit could run after the HIP runtime is gone; the slots are plain
// atomics, so no code of this library runs at exit).  Past READBACK_POOL
// concurrent calls the copy goes to pageable memory.
constexpr int READBACK_POOL = 64;
std::atomic<Readback *> g_readback_free[READBACK_POOL];
std::atomic<int> g_readback_made{0};

Readback *take_readback() {
    for (int i = 0; i < READBACK_POOL; ++i) {
        Readback *p = g_readback_free[i].exchange(nullptr, std::memory_order_acquire);
        if (p) return p;
    }
    if (g_readback_made.fetch_add(1, std::memory_order_relaxed) >= READBACK_POOL) {
        g_readback_made.fetch_sub(1, std::memory_order_relaxed);
        return nullptr;
    }
    void *p = nullptr;
    if (hipHostMalloc(&p, sizeof(Readback), hipHostMallocDefault) != hipSuccess) {
        g_readback_made.fetch_sub(1, std::memory_order_relaxed);
        return nullptr;
    }
    return static_cast<Readback *>(p);
}

void give_readback(Readback *p) {
    for (int i = 0; i < READBACK_POOL; ++i) {
        Readback *expected = nullptr;
        if (g_readback_free[i].compare_exchange_strong(expected, p, std::memory_order_release,
                                                       std::memory_order_relaxed))
            return;
    }
    // unreachable: at most READBACK_POOL buffers exist, each in one slot or in use
}

// Copies the control block back (the call's only device-to-host transfer)
// and synchronises the stream.  pool: through a pinned buffer of the pool;
// otherwise straight into *out (pageable), which allocates nothing.
nms_status read_back(const Work &w, hipStream_t stream, Readback *out, bool pool = true) {
    Readback *pin = pool ? take_readback() : nullptr;
    Readback *dst = pin ? pin : out;
    hipError_t e = hipMemcpyAsync(dst, w.ctrl, sizeof(Readback), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (pin) {
        if (e == hipSuccess) *out = *pin;
        give_readback(pin);
    }
    return hip_status(e);
}

// A pinned buffer of the pool, held for one call and given back on every
// way out; null when none is wanted or none is free.
struct PinnedSlot {
    Readback *p;
    explicit PinnedSlot(bool want) : p(want ? take_readback() : nullptr) {}
    ~PinnedSlot() {
        if (p) give_readback(p);
    }
    PinnedSlot(const PinnedSlot &) = delete;
    PinnedSlot &operator=(const PinnedSlot &) = delete;
    Post post(uint64_t tag) const { return Post{p, tag}; }
};

// How long the host spins on a posted result before it blocks in
// hipStreamSynchronize instead (a long call, or one queued behind other
// work on the stream).
constexpr double POST_SPIN_US = 2000.0;

// The end of a call.  With a pinned buffer: wait until the call's last
// kernel has posted its result there with `tag` (spinning, then blocking;
// a kernel that ended without posting is an internal error).  Without one:
// copy the control block's head back (pageable, allocates nothing) and
// synchronise the stream.
nms_status collect(const Work &w, hipStream_t stream, Readback *pin, uint64_t tag,
                   Readback *out) {
    if (pin == nullptr) {
        hipError_t e = hipMemcpyAsync(out, w.ctrl, sizeof(Readback), hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        return hip_status(e);
    }
    const auto t0 = std::chrono::steady_clock::now();
    while (__atomic_load_n(&pin->tag, __ATOMIC_ACQUIRE) != tag) {
        const double us =
            std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
        if (us > POST_SPIN_US) {
            const hipError_t e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_status(e);
            if (__atomic_load_n(&pin->tag, __ATOMIC_ACQUIRE) != tag) return NMS_HIP_ERROR;
            break;
        }
    }
    *out = *pin;
    return NMS_OK;
}

nms_status device_error(uint32_t err) {
    if (err & ERR_INTERNAL) return NMS_HIP_ERROR;
    if (err & ERR_BAD_BOXES) return NMS_BAD_BOXES;
    if (err & ERR_BAD_OFFSETS) return NMS_BAD_OFFSETS;
    if (err & ERR_NONFINITE) return NMS_NONFINITE_INPUT;
    return NMS_OK;
}

struct EventSet {
    hipEvent_t ev[NMS_NUM_STAGES + 1];
    bool made = false;
    bool create() {
        for (int i = 0; i <= NMS_NUM_STAGES; ++i) {
            if (hipEventCreate(&ev[i]) != hipSuccess) {
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
                return false;
            }
        }
        made = true;
        return true;
    }
    ~EventSet() {
        if (made)
            for (int i = 0; i <= NMS_NUM_STAGES; ++i) (void)hipEventDestroy(ev[i]);
    }
};

nms_status run_nms(const float *boxes, const float *scores, int64_t n, float thresh,
                   const int32_t *class_ids, const int64_t *offsets, int64_t num_images,
                   int64_t *keep_out, int64_t *num_kept, void *workspace, size_t ws_bytes,
                   void *stream_ptr, float *stage_ms, bool allow_fusion, bool one_launch,
                   bool pinned_pool = true, bool team_sort = true, bool sample_sort = true) {
    if (num_kept == nullptr) return NMS_INVALID_ARG;
    *num_kept = 0;
    if (stage_ms)
        for (int i = 0; i < NMS_NUM_STAGES; ++i) stage_ms[i] = 0.0f;
    nms_status st = check_common(n, thresh, offsets, num_images);
    if (st != NMS_OK) return st;
    if (n == 0) return NMS_OK;
    if (!boxes || !scores || !keep_out || !workspace) return NMS_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(boxes) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return NMS_INVALID_ARG;
    Layout L;
    make_layout(n, &L);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    // one image runs without dense mask rows first (see Problem::dense)
    Problem P = make_problem(boxes, scores, n, thresh, class_ids, offsets, num_images);
    P.team_sort = team_sort;
    P.sample_sort = team_sort && sample_sort;
    if (ws_bytes < (P.dense ? L.total : L.off_mask)) return NMS_WORKSPACE_TOO_SMALL;
    const Work w = carve(workspace, L);

    EventSet events;
    if (stage_ms && !events.create()) return NMS_HIP_ERROR;
    auto mark = [&](int i) -> hipError_t {
        return stage_ms ? hipEventRecord(events.ev[i], stream) : hipSuccess;
    };

    // only_mask: only the mask stage ran (the one launch, timed there)
    auto finish = [&](const Readback &rb, bool only_mask) -> nms_status {
        const nms_status ds = device_error(rb.error);
        if (ds != NMS_OK) return ds;
        if (stage_ms) {
            for (int i = 0; i < NMS_NUM_STAGES; ++i) {
                if (only_mask && i != NMS_STAGE_MASK) continue;
                float ms = 0.0f;
                if (hipEventElapsedTime(&ms, events.ev[i], events.ev[i + 1]) != hipSuccess)
                    return NMS_HIP_ERROR;
                stage_ms[i] = ms;
            }
        }
        *num_kept = rb.count;
        return NMS_OK;
    };

    // The result comes back through a pinned buffer of the pool, posted by
    // the call's last kernel; profiled calls copy it back and synchronise
    // (their events must have completed).
    const PinnedSlot slot(pinned_pool && stage_ms == nullptr);

    hipError_t e = hipSuccess;
    // One small image: the whole call in one launch (timed as the mask
    // stage).  Its result stands once its sweep finished, and an input
    // error stands as it is; otherwise the stages below run from the start.
    if (one_launch && small_launch_applies(P)) {
        const uint64_t tag = next_epoch();
        for (int i = 0; i <= 2 && e == hipSuccess; ++i) e = mark(i);
        if (e == hipSuccess)
            e = launch_small(P, L, w, keep_out, next_epoch(), slot.post(tag), stream);
        for (int i = 3; i <= NMS_NUM_STAGES && e == hipSuccess; ++i) e = mark(i);
        if (e != hipSuccess) return NMS_HIP_ERROR;
        Readback rb;
        st = collect(w, stream, slot.p, tag, &rb);
        if (st != NMS_OK) return st;
        if (rb.sweep_done == 1u || rb.error != 0u) return finish(rb, true);
    }

    for (;;) {
    const uint64_t tag = next_epoch();
    e = mark(0);
    if (e == hipSuccess) e = launch_radix_sort(P, L, w, next_epoch(), stream);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = mark(2);
    // One image of moderate size: the sweep runs inside the mask launch and
    // posts the result.
    const bool fused = allow_fusion && fused_launch_applies(P, L);
    if (e == hipSuccess)
        e = fused ? launch_mask_sweep(P, L, w, keep_out, stream, slot.post(tag))
                  : launch_mask(P, L, w, stream);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess && P.grouped) e = launch_group_sweep(P, L, w, stream);
    // one image: otherwise the sweep is the last kernel and posts the result
    if (e == hipSuccess && !fused)
        e = launch_sweep(P, L, w, keep_out, stream,
                         P.grouped ? Post{nullptr, 0} : slot.post(tag));
    if (e == hipSuccess) e = mark(4);
    if (e == hipSuccess && P.grouped) e = launch_compact(P, L, w, keep_out, stream);
    if (e == hipSuccess && P.grouped) e = launch_publish(w, slot.post(tag), stream);
    if (e == hipSuccess) e = mark(5);
    if (e != hipSuccess) return NMS_HIP_ERROR;

    Readback rb;
    st = collect(w, stream, slot.p, tag, &rb);
    if (st != NMS_OK) return st;
    // the fused sweep stopped without a result: the plain sweep on the
    // finished mask (it posts under a new tag)
    if (fused && rb.sweep_done != 1u && rb.error == 0u && (rb.flags & FLAG_SORT_RETRY) == 0u) {
        const uint64_t tag2 = next_epoch();
        if (launch_sweep(P, L, w, keep_out, stream, slot.post(tag2)) != hipSuccess)
            return NMS_HIP_ERROR;
        st = collect(w, stream, slot.p, tag2, &rb);
        if (st != NMS_OK) return st;
    }
    // the sample sort's buckets overflowed: again, with the radix passes
    if ((rb.flags & FLAG_SORT_RETRY) != 0u && rb.error == 0u && P.sample_sort) {
        P.sample_sort = false;
        continue;
    }
    if (P.dense || (rb.flags & FLAG_NEEDS_DENSE) == 0u || rb.error != 0u) return finish(rb, false);
    // a row tile's list overflowed: again, with dense rows, if they fit
    if (ws_bytes < L.total) return NMS_WORKSPACE_TOO_SMALL;
    P.dense = true;
    }
}

// Matrix NMS: the same sort, then prep, overlap maximum, decay test, kept
// bitmap and the score-order compaction.  Stage times (when asked): sort,
// overlap maximum, decay test + compaction.
nms_status run_matrix(const float *boxes, const float *scores, int64_t n, float score_thresh,
                      double sigma, int64_t *keep_out, int64_t *num_kept, void *workspace,
                      size_t ws_bytes, void *stream_ptr, float *stage_ms) {
    if (num_kept == nullptr) return NMS_INVALID_ARG;
    *num_kept = 0;
    if (stage_ms)
        for (int i = 0; i < NMS_MATRIX_NUM_STAGES; ++i) stage_ms[i] = 0.0f;
    if (n < 0 || std::isnan(score_thresh) || !std::isfinite(sigma) || !(sigma > 0.0))
        return NMS_INVALID_ARG;
    if (n > NMS_MAX_BOXES) return NMS_TOO_LARGE;
    if (n == 0) return NMS_OK;
    if (!boxes || !scores || !keep_out || !workspace) return NMS_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(boxes) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return NMS_INVALID_ARG;
    Layout L;
    make_layout(n, &L);
    if (ws_bytes < L.off_mask) return NMS_WORKSPACE_TOO_SMALL;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    const Problem P = make_problem(boxes, scores, n, score_thresh, nullptr, nullptr, 0);
    const Work w = carve(workspace, L);

    EventSet events;
    if (stage_ms && !events.create()) return NMS_HIP_ERROR;
    auto mark = [&](int i) -> hipError_t {
        return stage_ms ? hipEventRecord(events.ev[i], stream) : hipSuccess;
    };
    hipError_t e = mark(0);
    if (e == hipSuccess) e = launch_radix_sort(P, L, w, next_epoch(), stream);
    if (e == hipSuccess) e = launch_matrix_prep(P, L, w, sigma, stream);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = launch_matrix_overlap_max(P, L, w, stream);
    if (e == hipSuccess) e = mark(2);
    const PinnedSlot slot(stage_ms == nullptr);
    const uint64_t tag = next_epoch();
    if (e == hipSuccess) e = launch_matrix_decay(P, L, w, sigma, stream);
    if (e == hipSuccess) e = launch_compact(P, L, w, keep_out, stream);
    if (e == hipSuccess) e = launch_publish(w, slot.post(tag), stream);
    if (e == hipSuccess) e = mark(3);
    if (e != hipSuccess) return NMS_HIP_ERROR;

    Readback rb;
    nms_status st = collect(w, stream, slot.p, tag, &rb);
    if (st != NMS_OK) return st;
    st = device_error(rb.error);
    if (st != NMS_OK) return st;
    if (stage_ms) {
        for (int i = 0; i < NMS_MATRIX_NUM_STAGES; ++i) {
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, events.ev[i], events.ev[i + 1]) != hipSuccess)
                return NMS_HIP_ERROR;
            stage_ms[i] = ms;
        }
    }
    *num_kept = rb.count;
    return NMS_OK;
}

// Scratch of nms_f32_static: the workspace of one call, in a file-scope
// device array.  Each device the library runs on holds its own copy (the HIP
// runtime allocates it with the code object); host code may not use the
// array's name as an address, only the pointer hipGetSymbolAddress returns
// for the device, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[NMS_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void *> g_scratch_ptr[MAX_DEVICES];

// The current device's scratch address, or nullptr (with *status set).
void *static_scratch(nms_status *status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        *status = NMS_HIP_ERROR;
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // two threads may both look it up; they get the same address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            *status = NMS_HIP_ERROR;
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace
}  // namespace gnms

using namespace gnms;

extern "C" {

nms_status nms_workspace_size(int64_t n, int64_t num_images, int has_classes, size_t *bytes) {
    (void)num_images;
    (void)has_classes;
    if (bytes == nullptr || n < 0) return NMS_INVALID_ARG;
    if (n > NMS_MAX_BOXES) return NMS_TOO_LARGE;
    Layout L;
    make_layout(n, &L);
    *bytes = L.total;
    return NMS_OK;
}

nms_status nms_workspace_size_lists(int64_t n, size_t *bytes) {
    if (bytes == nullptr || n < 0) return NMS_INVALID_ARG;
    if (n > NMS_MAX_BOXES) return NMS_TOO_LARGE;
    Layout L;
    make_layout(n, &L);
    *bytes = L.off_mask;
    return NMS_OK;
}

nms_status nms_f32(const float *boxes, const float *scores, int64_t n, float iou_thresh,
                   const int32_t *class_ids, const int64_t *batch_offsets, int64_t num_images,
                   int64_t *keep_out, int64_t *num_kept, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return run_nms(boxes, scores, n, iou_thresh, class_ids, batch_offsets, num_images, keep_out,
                   num_kept, workspace, workspace_bytes, stream, nullptr, true, false);
}

nms_status nms_f32_ex(const float *boxes, const float *scores, int64_t n, float iou_thresh,
                      const int32_t *class_ids, const int64_t *batch_offsets, int64_t num_images,
                      int64_t *keep_out, int64_t *num_kept, void *workspace,
                      size_t workspace_bytes, void *stream, int flags) {
    if (num_kept != nullptr) *num_kept = 0;
    if ((flags & ~(NMS_FLAG_ONE_LAUNCH | NMS_FLAG_PASS_SORT | NMS_FLAG_RADIX_SORT)) != 0)
        return NMS_INVALID_ARG;
    return run_nms(boxes, scores, n, iou_thresh, class_ids, batch_offsets, num_images, keep_out,
                   num_kept, workspace, workspace_bytes, stream, nullptr, true,
                   (flags & NMS_FLAG_ONE_LAUNCH) != 0, true, (flags & NMS_FLAG_PASS_SORT) == 0,
                   (flags & NMS_FLAG_RADIX_SORT) == 0);
}

nms_status nms_f32_static(const float *boxes, const float *scores, int64_t n, float iou_thresh,
                          const int32_t *class_ids, const int64_t *batch_offsets,
                          int64_t num_images, int64_t *keep_out, int64_t *num_kept,
                          void *stream) {
    if (num_kept == nullptr) return NMS_INVALID_ARG;
    *num_kept = 0;
    nms_status st = check_common(n, iou_thresh, batch_offsets, num_images);
    if (st != NMS_OK) return st;
    if (n > NMS_STATIC_MAX_BOXES) return NMS_TOO_LARGE;
    if (n == 0) return NMS_OK;
    Layout L;
    make_layout(n, &L);
    if (L.total > (size_t)NMS_STATIC_SCRATCH_BYTES) return NMS_TOO_LARGE;
    void *ws = static_scratch(&st);
    if (ws == nullptr) return st;
    // the same kernels as nms_f32 on the static scratch; the read-back goes
    // to the caller's stack (pageable), so nothing is allocated
    return run_nms(boxes, scores, n, iou_thresh, class_ids, batch_offsets, num_images, keep_out,
                   num_kept, ws, (size_t)NMS_STATIC_SCRATCH_BYTES, stream, nullptr, true, false,
                   false);
}

nms_status nms_f32_profiled(const float *boxes, const float *scores, int64_t n,
                            float iou_thresh, const int32_t *class_ids,
                            const int64_t *batch_offsets, int64_t num_images,
                            int64_t *keep_out, int64_t *num_kept, void *workspace,
                            size_t workspace_bytes, void *stream, float *stage_ms,
                            int flags) {
    const int known = NMS_PROFILE_NO_FUSION | NMS_PROFILE_ONE_LAUNCH | NMS_PROFILE_PASS_SORT |
                      NMS_PROFILE_RADIX_SORT;
    const int both = NMS_PROFILE_NO_FUSION | NMS_PROFILE_ONE_LAUNCH;
    if (stage_ms == nullptr || (flags & ~known) != 0 || (flags & both) == both)
        return NMS_INVALID_ARG;
    return run_nms(boxes, scores, n, iou_thresh, class_ids, batch_offsets, num_images, keep_out,
                   num_kept, workspace, workspace_bytes, stream, stage_ms,
                   (flags & NMS_PROFILE_NO_FUSION) == 0, (flags & NMS_PROFILE_ONE_LAUNCH) != 0,
                   true, (flags & NMS_PROFILE_PASS_SORT) == 0,
                   (flags & NMS_PROFILE_RADIX_SORT) == 0);
}

nms_status nms_matrix_workspace_size(int64_t n, size_t *bytes) {
    if (bytes == nullptr || n < 0) return NMS_INVALID_ARG;
    if (n > NMS_MAX_BOXES) return NMS_TOO_LARGE;
    Layout L;
    make_layout(n, &L);
    *bytes = L.off_mask;
    return NMS_OK;
}

nms_status nms_matrix_f32(const float *boxes, const float *scores, int64_t n, float score_thresh,
                          double sigma, int64_t *keep_out, int64_t *num_kept, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return run_matrix(boxes, scores, n, score_thresh, sigma, keep_out, num_kept, workspace,
                      workspace_bytes, stream, nullptr);
}

nms_status nms_matrix_f32_profiled(const float *boxes, const float *scores, int64_t n,
                                   float score_thresh, double sigma, int64_t *keep_out,
                                   int64_t *num_kept, void *workspace, size_t workspace_bytes,
                                   void *stream, float *stage_ms) {
    if (stage_ms == nullptr) return NMS_INVALID_ARG;
    return run_matrix(boxes, scores, n, score_thresh, sigma, keep_out, num_kept, workspace,
                      workspace_bytes, stream, stage_ms);
}

const char *nms_status_string(nms_status status) {
    switch (status) {
        case NMS_OK: return "NMS_OK";
        case NMS_INVALID_ARG: return "NMS_INVALID_ARG";
        case NMS_WORKSPACE_TOO_SMALL: return "NMS_WORKSPACE_TOO_SMALL";
        case NMS_NONFINITE_INPUT: return "NMS_NONFINITE_INPUT";
        case NMS_BAD_OFFSETS: return "NMS_BAD_OFFSETS";
        case NMS_TOO_LARGE: return "NMS_TOO_LARGE";
        case NMS_HIP_ERROR: return "NMS_HIP_ERROR";
        case NMS_BAD_BOXES: return "NMS_BAD_BOXES";
    }
    return "NMS_UNKNOWN_STATUS";
}

nms_status nms_debug_order(const float *scores, int64_t n, const int32_t *class_ids,
                           const int64_t *batch_offsets, int64_t num_images,
                           int32_t *order_out, int32_t *score_order_out, void *workspace,
                           size_t workspace_bytes, void *stream_ptr) {
    nms_status st = check_common(n, 0.5f, batch_offsets, num_images);
    if (st != NMS_OK) return st;
    if (n == 0) return NMS_OK;
    if (!scores || !order_out || !workspace) return NMS_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NMS_INVALID_ARG;
    Layout L;
    make_layout(n, &L);
    if (workspace_bytes < L.total) return NMS_WORKSPACE_TOO_SMALL;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    Problem P = make_problem(nullptr, scores, n, 0.5f, class_ids, batch_offsets, num_images);
    P.sample_sort = true;
    const Work w = carve(workspace, L);
    for (;;) {
    hipError_t e = launch_radix_sort(P, L, w, next_epoch(), stream);
    Readback rb;
    if (e == hipSuccess) {
        st = read_back(w, stream, &rb);
        if (st != NMS_OK) return st;
        if ((rb.flags & FLAG_SORT_RETRY) != 0u && rb.error == 0u && P.sample_sort) {
            P.sample_sort = false;  // the sample sort's buckets overflowed
            continue;
        }
    }
    if (e == hipSuccess)
        e = hipMemcpyAsync(order_out, w.order, (size_t)n * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess && score_order_out) {
        if (P.grouped)
            e = hipMemcpyAsync(score_order_out, w.score_order, (size_t)n * 4,
                               hipMemcpyDeviceToDevice, stream);
        else
            e = hipMemcpyAsync(score_order_out, w.order, (size_t)n * 4,
                               hipMemcpyDeviceToDevice, stream);
    }
    if (e != hipSuccess) return NMS_HIP_ERROR;
    if (hipStreamSynchronize(stream) != hipSuccess) return NMS_HIP_ERROR;
    return device_error(rb.error);
    }
}

nms_status nms_debug_mask(const float *boxes, const float *scores, int64_t n,
                          float iou_thresh, const int32_t *class_ids,
                          const int64_t *batch_offsets, int64_t num_images,
                          uint64_t *mask_out, int32_t *order_out, void *workspace,
                          size_t workspace_bytes, void *stream_ptr) {
    nms_status st = check_common(n, iou_thresh, batch_offsets, num_images);
    if (st != NMS_OK) return st;
    if (n == 0) return NMS_OK;
    if (!boxes || !scores || !mask_out || !workspace) return NMS_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(boxes) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return NMS_INVALID_ARG;
    Layout L;
    make_layout(n, &L);
    if (workspace_bytes < L.total) return NMS_WORKSPACE_TOO_SMALL;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    Problem P = make_problem(boxes, scores, n, iou_thresh, class_ids, batch_offsets, num_images);
    P.dense = true;  // the export reads the dense rows
    P.sample_sort = true;
    const Work w = carve(workspace, L);
    for (;;) {
    hipError_t e = launch_radix_sort(P, L, w, next_epoch(), stream);
    if (e == hipSuccess) {
        Readback rs;
        st = read_back(w, stream, &rs);
        if (st != NMS_OK) return st;
        if ((rs.flags & FLAG_SORT_RETRY) != 0u && rs.error == 0u && P.sample_sort) {
            P.sample_sort = false;  // the sample sort's buckets overflowed
            continue;
        }
    }
    if (e == hipSuccess) e = launch_mask(P, L, w, stream);
    if (e == hipSuccess) e = launch_expand_mask(P, L, w, mask_out, stream);
    if (e == hipSuccess && order_out)
        e = hipMemcpyAsync(order_out, w.order, (size_t)n * 4, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return NMS_HIP_ERROR;
    Readback rb;
    st = read_back(w, stream, &rb);
    if (st != NMS_OK) return st;
    return device_error(rb.error);
    }
}

nms_status nms_debug_plan(int64_t n, int64_t num_images, int has_classes, int32_t *plan) {
    if (plan == nullptr || n < 0 || num_images < 0) return NMS_INVALID_ARG;
    if (n > NMS_MAX_BOXES) return NMS_TOO_LARGE;
    for (int i = 0; i < NMS_PLAN_FIELDS; ++i) plan[i] = -1;
    if (n == 0) return NMS_OK;
    Layout L;
    make_layout(n, &L);
    Problem P = make_problem(nullptr, nullptr, n, 0.5f, nullptr, nullptr, num_images);
    P.grouped = has_classes != 0 || num_images > 1;
    P.strip = P.grouped ? STRIP_GROUPED : STRIP_SINGLE;
    const bool fused = fused_launch_applies(P, L);
    plan[NMS_PLAN_MASK_QSHIFT] = separate_mask_qshift(P, L);
    plan[NMS_PLAN_FUSED] = fused ? 1 : 0;
    plan[NMS_PLAN_FUSED_QSHIFT] = fused ? fused_mask_qshift(P, L) : -1;
    plan[NMS_PLAN_RANK_SORT] = (!P.grouped && n <= RANK_SORT_MAX) ? 1 : 0;
    plan[NMS_PLAN_SMALL] = small_launch_applies(P) ? 1 : 0;
    plan[NMS_PLAN_TEAM_SORT] = L.off_team != 0 && team_sort_applies(P) ? 1 : 0;
    plan[NMS_PLAN_SAMPLE_SORT] = L.off_team != 0 && team_sample_applies(P) ? 1 : 0;
    return NMS_OK;
}

nms_status nms_debug_decide(const float *inter, const float *uni, int64_t count,
                            float iou_thresh, int all_positive_areas, uint8_t *out,
                            void *stream_ptr) {
    if (count < 0 || std::isnan(iou_thresh)) return NMS_INVALID_ARG;
    if (count == 0) return NMS_OK;
    if (!inter || !uni || !out) return NMS_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    hipError_t e =
        launch_decide(inter, uni, count, iou_thresh, all_positive_areas != 0, out, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return hip_status(e);
}

}  // extern "C"
