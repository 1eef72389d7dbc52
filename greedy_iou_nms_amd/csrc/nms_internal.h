// Internal declarations shared by the HIP translation units of libgreedy_nms.
// Nothing here is part of the public ABI (include/greedy_nms.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gnms {

// Error bits raised on the device (Ctrl::error).
constexpr uint32_t ERR_NONFINITE = 1u;
constexpr uint32_t ERR_BAD_OFFSETS = 2u;
constexpr uint32_t ERR_INTERNAL = 4u;  // a bounded wait inside a kernel gave up
constexpr uint32_t ERR_BAD_BOXES = 8u;  // Matrix NMS: a box with x1 > x2 or y1 > y2

// Ctrl::flags bits.
// every box has x1 < x2, y1 < y2 and a finite area > 0
constexpr uint32_t FLAG_ORDERED_BOXES = 1u;
// Matrix NMS: some child with a negative score at or above the threshold,
// for which a father with no overlap can still decide the decay test.
constexpr uint32_t FLAG_MATRIX_ZERO_PAIRS_MATTER = 2u;
// One image without dense mask rows: a row tile had more nonzero mask words
// than its list holds, so the sweep stopped without a result; the call has
// to run again with dense rows.
constexpr uint32_t FLAG_NEEDS_DENSE = 4u;
// One image sorted by sample sort: a bucket held more boxes than one
// workgroup sorts in LDS, so the sorted arrays are incomplete; the call runs
// again with the radix passes.
constexpr uint32_t FLAG_SORT_RETRY = 8u;

// Per-call control block at the start of the workspace.  The sort kernel
// initialises it; later kernels read plan fields and raise error bits.  The
// first 32 bytes (Readback) reach the host at the end of a call.
struct Ctrl {
    uint32_t error;
    uint32_t flags;
    int32_t count;          // kept boxes
    int32_t num_items;      // mask work items (row tile x strip)
    int32_t band_stride;    // mask row stride in 64-bit words
    int32_t num_segments;   // groups present (1 for a single image)
    // 1 once a sweep that may give up (the fused single-image sweep, the
    // parallel grouped sweep) finished; the plain sweep kernel then returns
    uint32_t sweep_done;
    int32_t reserved[9];
};
static_assert(sizeof(Ctrl) == 64, "Ctrl layout");

// The head of the control block as the host reads it at the end of a call,
// and the call's tag (see Post).  A plain copy of the control block fills
// the first eight fields.
struct Readback {
    uint32_t error;
    uint32_t flags;
    int32_t count;
    int32_t num_items;
    int32_t band_stride;
    int32_t num_segments;
    uint32_t sweep_done;
    int32_t reserved0;
    uint64_t tag;
};

// Where the last kernel of a call posts the result: a pinned host buffer
// (null: nothing is posted and the host copies the control block back) and
// the call's tag.  The tag is stored last, with release semantics at system
// scope, and the host spins on it: it then sees the other fields complete,
// with no copy to enqueue and no stream synchronisation, which cost about
// 8 us more per call on this GPU.
struct Post {
    Readback *dst;
    uint64_t tag;
};

// One thread posts the control block's head.  Every store the host relies on
// (the output indices) must have completed before: the kernel's waves wait
// for their stores and meet at a barrier first.  valid = false posts a
// result that says only "no result" (sweep_done 0, no error), for a kernel
// that gave up before the control block was complete.
__device__ __forceinline__ void post_result(const Post &p, const Ctrl *ctrl, bool valid = true) {
    if (p.dst == nullptr) return;
    auto ld = [](const auto *q) {
        return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    Readback *d = p.dst;
    d->error = valid ? ld(&ctrl->error) : 0u;
    d->flags = valid ? ld(&ctrl->flags) : 0u;
    d->count = valid ? ld(&ctrl->count) : 0;
    d->num_items = valid ? ld(&ctrl->num_items) : 0;
    d->band_stride = valid ? ld(&ctrl->band_stride) : 0;
    d->num_segments = valid ? ld(&ctrl->num_segments) : 0;
    d->sweep_done = valid ? ld(&ctrl->sweep_done) : 0u;
    d->reserved0 = 0;
    __hip_atomic_store(&d->tag, p.tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Column tiles per mask work item ("strip"): 16 for one image, 4 for grouped
// input whose bands are only a few tiles wide.
constexpr int STRIP_SINGLE = 8;
constexpr int STRIP_GROUPED = 4;

// Multi-workgroup radix sort (one image): a workgroup of RADIX_THREADS ranks
// one tile of RADIX_TILE keys per pass.
constexpr int RADIX_THREADS = 256;
constexpr int RADIX_E = 8;
constexpr int RADIX_TILE = RADIX_THREADS * RADIX_E;
// One image of at most this many boxes is sorted by ranking: every box
// counts the boxes that precede it (the keys of all boxes fit in LDS).
constexpr int RANK_SORT_MAX = 16384;
// 8-bit digit passes: 4 on the score key, then (grouped input) 4 on the
// class key and 4 on the image.
constexpr int RADIX_PASSES = 12;
// The radix sort in one launch (team_sort.hip): up to TEAM_MAX resident
// workgroups of TEAM_THREADS threads, each ranking a tile of up to
// TEAM_EMAX boxes per thread in every pass; blocks beside the team check.
constexpr int TEAM_THREADS = 1024;
constexpr int TEAM_MAX = 32;
constexpr int TEAM_EMAX = 4;
constexpr int64_t TEAM_MAX_N = (int64_t)TEAM_MAX * TEAM_THREADS * TEAM_EMAX;
// Checker blocks per team member at most (the team's XCD and up to seven
// others).
constexpr int TEAM_CHECKERS_PER_MEMBER = 7;
// Team members the workspace of n boxes provides for: the most any device
// can use (tiles of at least TEAM_THREADS boxes).
constexpr int64_t team_layout_members(int64_t n) {
    return n < 1 ? 0 : ((n + TEAM_THREADS - 1) / TEAM_THREADS < TEAM_MAX
                            ? (n + TEAM_THREADS - 1) / TEAM_THREADS
                            : TEAM_MAX);
}
// Bytes of the team's tagged words for tl members (carved by team_work in
// team_sort.hip in this order): tile counts and prefixes [tl][RADIX_PASSES
// * 256], totals [RADIX_PASSES * 256], per-pass tile counts [RADIX_PASSES]
// [tl][256], done and extent slots [tl][16], checker slots
// [tl * TEAM_CHECKERS_PER_MEMBER][16].
constexpr size_t team_ws_bytes(int64_t tl) {
    return 8 * ((size_t)2 * tl * RADIX_PASSES * 256 + (size_t)RADIX_PASSES * 256 +
                (size_t)RADIX_PASSES * tl * 256 + (size_t)2 * tl * 16 +
                (size_t)tl * TEAM_CHECKERS_PER_MEMBER * 16);
}

// Per radix pass, decided on the device from the digit counts.
struct RadixPassPlan {
    uint32_t skip;        // every key has the same digit: the pass moves nothing
    uint32_t src;         // which of the two key/value buffers the pass reads
    uint32_t last;        // the last pass that runs: writes the sorted arrays
    uint32_t last_score;  // the last score pass that runs: writes the score order
};
constexpr int SWEEP_THREADS = 512;
// Grouped compaction: score ranks per workgroup.
constexpr int COMPACT_CHUNK = 2048;
// Grouped sweep: one wave per segment keeps the removed words of the next
// GROUP_SWEEP_WIN row tiles; wider bands fall back to the plain sweep.
constexpr int GROUP_SWEEP_WIN = 256;
constexpr int MASK_THREADS = 256;

// Nonzero mask words recorded per row tile (row, word index, value) besides
// the dense rows.  A tile with more nonzero words than this is flagged by its
// count exceeding the capacity, and the sweep reads the dense rows of its
// kept boxes instead.
constexpr int TILE_LIST_CAP = 2048;

// Words of a row that the sweep's resolver applies itself: the row's own
// tile (j = 0) and the next NEAR_TILES tiles.  They are copied, transposed,
// into tnear so that the 64 rows of a tile read word j with one coalesced
// load.  Words further right are applied by helper waves from the lists.
constexpr int NEAR_TILES = 4;
// Quantised overlap pre-test (one image sorted by the radix passes or the
// sample sort).  The sort quantises every sorted box's coordinates to
// 0 .. PACK_QMAX - 1 on a grid over the extent of all boxes (q rounds down,
// so it never reverses an order of two coordinates) and keeps 7 bits of each.
constexpr uint32_t PACK_QMAX = 32767u;
// The coarse pre-test: the grid cut to 7 bits (v = min(q >> 8, 126), which
// never reverses an order either) and all four comparisons of
// a pair in one 32-bit subtraction, one byte each.  A box's column word and
// row word are
//   col = (0xFF - vx2) | (0x7F + vx1) << 8 | (0xFF - vy2) << 16 | (0x7F + vy1) << 24
//   row = (0x80 - vx1) | vx2 << 8          | (0x80 - vy1) << 16 | vy2 << 24
// (v of the raw coordinates, right and bottom edges included).  Every byte of
// col_c - row_r lies in 1 .. 0xFD, so no byte borrows from the next, and its
// bit 7 is set iff vx1_r > vx2_c (byte 0), vx1_c > vx2_r (byte 1), or the same
// for y: an order of the coordinates that rules the overlap out.  Columns that
// take no part hold COARSE_NONE, whose byte 1 (0xFE) sets bit 7 against any
// row (vx2 <= 126).
constexpr uint32_t COARSE_SIGNS = 0x80808080u;
constexpr uint32_t COARSE_NONE = 0x7F80FE80u;
// Rows past n hold COARSE_NO_ROW: its byte 0 (1) sets bit 7 against every
// column (byte 0 of a column word is at least 0x81, of COARSE_NONE 0x80 with
// byte 1 set anyway), so a padding row never passes.
constexpr uint32_t COARSE_NO_ROW = 0x00000001u;

// Largest grid (in threads) a launch uses; kernels loop over what lies past it.
constexpr int64_t MAX_GRID_THREADS = (int64_t)1 << 31;

// One image with FUSE_MIN_WORDS .. FUSE_MAX_WORDS row tiles runs the mask
// and the sweep in one launch (the sweep's workgroup overlaps the mask's).
// Below the minimum the mask's items all finish at about the same time and
// there is nothing to overlap; above the maximum the sweep's LDS (removed
// bitmap) would no longer fit beside two mask workgroups per CU.
constexpr int FUSE_MIN_WORDS = 512;
constexpr int FUSE_MAX_WORDS = 4096;
// One image of at most this many boxes runs sort, mask, sweep and output in
// one launch.
constexpr int SMALL_MAX = 4096;

// Workspace carve-up, computed on the host from n alone.
struct Layout {
    int64_t n = 0;
    int64_t words = 0;      // W = ceil(n / 64): words per full mask row, row tiles
    int64_t npad = 0;       // 64 * W
    int64_t mstride = 0;    // worst-case mask row stride in words
    int64_t tiles = 0;      // radix-sort tiles, ceil(npad / RADIX_TILE)
    size_t off_ctrl = 0, off_keys0 = 0, off_keys1 = 0, off_vals0 = 0, off_vals1 = 0;
    size_t off_order = 0, off_score_order = 0, off_seg = 0, off_inv = 0;
    size_t off_sb = 0, off_area = 0, off_tile_cend = 0, off_item_base = 0, off_kept = 0;
    size_t off_tcount = 0, off_tent_wk = 0, off_tent_val = 0, off_tnear = 0;
    size_t off_hist_tile = 0, off_lb_status = 0, off_err_tile = 0;
    size_t off_gcls = 0, off_gimg = 0, off_pass_plan = 0, off_gbase = 0;
    size_t off_done = 0, off_seg_start = 0, off_start_bits = 0, off_block_cnt = 0;
    size_t off_momax = 0, off_mscore = 0, off_mlo = 0, off_mhi = 0, off_mdrop = 0;
    size_t off_tile_ext = 0, off_coarse = 0, off_arrive = 0;
    size_t off_team = 0;       // 0: no team sort for this n
    size_t off_team_ring = 0;  // the team's pass buffers: 3 x 2 x npad tagged words
    // the suppression bitmask comes last: Matrix NMS uses everything before it
    size_t off_mask = 0, total = 0;
};

bool make_layout(int64_t n, Layout *out);

// Device pointers into one workspace.
struct Work {
    Ctrl *ctrl;
    uint32_t *keys0, *keys1, *vals0, *vals1;
    int32_t *order;        // sorted position -> input index (group order)
    int32_t *score_order;  // score rank -> input index (grouped input only)
    uint32_t *seg;         // sorted position -> segment id (grouped input only)
    int32_t *inv;          // input index -> sorted position (grouped input only)
    float4 *sb;            // sorted boxes, padded to npad
    float *area;           // sorted areas, padded to npad
    int32_t *tile_cend;    // per row tile: one past the last column tile of its band
    int32_t *item_base;    // per row tile: first mask work item; [W] = total
    uint64_t *kept;        // W words: bit p = sorted position p kept
    uint32_t *tcount;      // per row tile: nonzero mask words in its 64 rows
    // per row tile r, entries [r * TILE_LIST_CAP, ...): (word << 6 | row in tile)
    uint32_t *tent_wk;
    uint64_t *tent_val;    // the word's value
    // [j][p] for j = 0..NEAR_TILES: row p's mask word for tile (p / 64) + j,
    // 0 where that tile lies outside the row's band
    uint64_t *tnear;
    uint64_t *mask;        // suppression bitmask rows
    // radix sort: per-tile digit histograms [tile][RADIX_PASSES][256],
    // look-back status words [pass][tile][256], per-tile
    // error bits from key generation, the grouped keys of every input box
    // (class key, image), and per pass its plan and digit starts [pass][256]
    uint32_t *hist_tile;
    uint32_t *lb_status;
    uint32_t *err_tile;
    uint32_t *gcls;
    uint32_t *gimg;
    RadixPassPlan *pass_plan;
    uint32_t *gbase;
    // fused mask + sweep: per row tile, mask work items finished
    uint32_t *done;
    // grouped: first sorted position of every segment, then n; bit p of
    // start_bits: a segment starts at sorted position p
    int32_t *seg_start;
    uint64_t *start_bits;
    // grouped compaction: kept boxes per block of COMPACT_CHUNK score ranks
    uint32_t *block_cnt;
    // Matrix NMS, per sorted position: the largest overlap with a father
    // (float bits), the score, the bounds of the decay test's fast path; and
    // per row tile the drop bits
    uint32_t *momax;
    float *mscore;
    double *mlo, *mhi;
    uint64_t *mdrop;
    // one image sorted by radix passes: per radix tile the extent of its
    // boxes (min x1, min y1, max x2, max y2); one image sorted by radix
    // passes or sample sort: per sorted position the column and row words
    // of the coarse pre-test (see COARSE_*; npad words each, srow after scol)
    float4 *tile_ext;
    uint32_t *scol, *srow;
    // one launch for small inputs: W + 1 slots, each the epoch of the last
    // call whose preparing workgroup finished
    uint64_t *arrive;
    // the radix sort in one launch: the team's tagged words and its ring of
    // pass buffers (null when the layout has none)
    uint64_t *team;
    uint64_t *team_ring;
};

Work carve(void *workspace, const Layout &L);

struct Problem {
    const float *boxes;
    const float *scores;
    int n;
    float thresh;
    const int32_t *class_ids;
    const int64_t *offsets;
    int num_images;
    bool grouped;          // class_ids or more than one image
    int strip;             // STRIP_SINGLE or STRIP_GROUPED
    // The mask kernel writes dense rows (every band word) besides the lists
    // of nonzero words.  Grouped input always (its sweep reads them); one
    // image only when a row tile's list overflows, after a first run
    // without them stopped (FLAG_NEEDS_DENSE).  Without dense rows the
    // workspace ends where the dense rows would begin (Layout::off_mask).
    bool dense;
    // The sort may run in one launch (team_sort_applies); false: one launch
    // per radix pass, as for inputs too large for the team.
    bool team_sort;
    // One image of RANK_SORT_MAX + 1 to TEAM_MAX_N boxes is sorted by sample
    // sort in one launch (team_sample_applies) when set; a call whose buckets
    // overflow runs again without it (FLAG_SORT_RETRY).
    bool sample_sort;
};

// Stage launchers; all enqueue on `stream` and return the launch status.
// launch_radix_sort sorts, gathers the sorted boxes and (grouped input)
// plans the segments and the mask work.
hipError_t launch_radix_sort(const Problem &P, const Layout &L, const Work &w, uint64_t epoch,
                             hipStream_t stream);
// The sort in one launch (team_sort.hip) applies: grouped input of up to
// TEAM_MAX_N boxes, or one image of RANK_SORT_MAX + 1 to TEAM_MAX_N boxes,
// on a device with room for the team on one XCD.  epoch: new for every call.
bool team_sort_applies(const Problem &P);
bool team_sample_applies(const Problem &P);
hipError_t launch_team_sample(const Problem &P, const Layout &L, const Work &w, uint64_t epoch,
                              hipStream_t stream);
hipError_t launch_team_sort(const Problem &P, const Layout &L, const Work &w, uint64_t epoch,
                            hipStream_t stream);
// Matrix NMS after the sort (matrix.hip): scores, bounds and checks; the
// largest overlap of every box with its fathers; the decay test; the kept
// bitmap (then launch_compact writes the output).
hipError_t launch_matrix_prep(const Problem &P, const Layout &L, const Work &w, double sigma,
                              hipStream_t stream);
hipError_t launch_matrix_overlap_max(const Problem &P, const Layout &L, const Work &w,
                                     hipStream_t stream);
hipError_t launch_matrix_decay(const Problem &P, const Layout &L, const Work &w, double sigma,
                               hipStream_t stream);
hipError_t launch_mask(const Problem &P, const Layout &L, const Work &w, hipStream_t stream);
// post: set only when the sweep is the call's last kernel (one image).
hipError_t launch_sweep(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                        hipStream_t stream, const Post &post = Post{nullptr, 0});
// One workgroup posts the control block's head (after the call's last
// kernel, where that kernel has many workgroups).
hipError_t launch_publish(const Work &w, const Post &post, hipStream_t stream);
// One image with FUSE_MIN_WORDS <= L.words <= FUSE_MAX_WORDS: mask and
// sweep in one launch, whose sweep workgroup posts the result.  A result
// with sweep_done clear and no error (a tile's list overflowed, or the mask
// took too long) means the sweep stopped: launch_sweep on the finished mask
// then does the work and posts again.
hipError_t launch_mask_sweep(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                             hipStream_t stream, const Post &post);

// Compute units of the current device (cached per device).
int device_cu_count();
// Row-group split (log2) the mask launch takes on the current device: as a
// separate launch, and as the fused mask + sweep launch.
int separate_mask_qshift(const Problem &P, const Layout &L);
int fused_mask_qshift(const Problem &P, const Layout &L);
// nms_f32 runs mask and sweep in one launch (one image of FUSE_MIN_WORDS to
// FUSE_MAX_WORDS row tiles whose mask takes the pre-test form).
bool fused_launch_applies(const Problem &P, const Layout &L);
// One image of 1 .. SMALL_MAX boxes: the whole call in one launch.  The
// result stands only if the control block's sweep_done reads 1 afterwards;
// otherwise (a wait gave up, a tile's list overflowed) the call runs the
// multi-launch path from the start.  epoch: new for every call.
bool small_launch_applies(const Problem &P);
hipError_t launch_small(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                        uint64_t epoch, const Post &post, hipStream_t stream);
hipError_t launch_compact(const Problem &P, const Layout &L, const Work &w, int64_t *keep_out,
                          hipStream_t stream);
// Grouped input: sweep every segment with its own wave.  launch_sweep must
// still follow; it returns at once unless a band is wider than the window.
hipError_t launch_group_sweep(const Problem &P, const Layout &L, const Work &w,
                              hipStream_t stream);
hipError_t launch_expand_mask(const Problem &P, const Layout &L, const Work &w,
                              uint64_t *mask_out, hipStream_t stream);
hipError_t launch_decide(const float *inter, const float *uni, int64_t count, float thresh,
                         bool positive_areas, uint8_t *out, hipStream_t stream);

// Threshold constants for the mask kernel's division-free test (see mask.hip).
struct Threshold {
    float t;
    double mid;      // t + ulp(t)/2, exact in binary64
    bool odd;        // t's last significand bit is 1 (ties round away from t)
    bool exact_ok;   // t is finite and > 0: the division-free test applies
};
Threshold make_threshold(float t);

}  // namespace gnms
