/*
 * greedy_nms.h -- C ABI of the MI355X (gfx950) greedy IoU non-maximum
 * suppression library (libgreedy_nms.so).
 *
 * What the library computes.  Greedy NMS as described on "LeetCUDA 14-nms"
 * (introduction and "algorithm and data flow"): visit the boxes by score,
 * highest first, with equal scores in ascending input order (stable sort);
 * keep a box unless an already-kept box of its group overlaps it with
 * IoU > iou_thresh (strictly); return the kept boxes as their original input
 * indices (that page's bug-3 fix), int64, in visiting order.  A group is the
 * pair (image, class): boxes of different images or classes never suppress
 * each other (the class check of "YOLOv5 post-processing GPU port",
 * section 2.2, extended to images).  With several groups the result is one
 * list over all boxes in global score order, with global indices.
 *
 * The IoU is this float32 expression, one IEEE binary32 operation per step,
 * no fused multiply-add (none of the pages prints its IoU routine; this
 * expression is the one the library fixes):
 *     area  = (x2 - x1) * (y2 - y1)
 *     w     = max(min(x2i, x2j) - max(x1i, x1j), 0)
 *     h     = max(min(y2i, y2j) - max(y1i, y1j), 0)
 *     inter = w * h
 *     union = (area_i + area_j) - inter
 *     suppress  iff  inter / union > iou_thresh      (correctly rounded)
 * No clipping or reordering of coordinates is applied.
 *
 * Memory.  Every pointer argument named "device" is HIP device memory on the
 * current device; the caller allocates and owns every buffer (inputs, output,
 * workspace).  The library allocates no device memory, keeps no pointer to a
 * caller's buffer after a call returns and holds no device state between
 * calls, so calls on different streams with distinct workspaces may run
 * concurrently.  What the library does allocate, and keeps:
 *   - pinned host buffers of 40 bytes (hipHostMalloc) into which a call's
 *     last kernel posts the kept count, the device-detected errors and the
 *     call's tag: a process-wide pool of at most 64, one per call running at
 *     that moment, allocated when every existing one is in use and kept
 *     until the process ends (past 64 concurrent calls the call copies the
 *     control block back into pageable memory instead);
 *   - per profiled call (the *_profiled variants), HIP events, created and
 *     destroyed inside the call;
 *   - for nms_f32_static, a statically sized device array in the library's
 *     code object (see there).
 * No library code runs at process exit (no static or thread-local object
 * has a destructor).
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  All work
 * is enqueued on it.  Each nms_* compute call returns once its result is
 * complete: its last kernel posts the result into a pinned buffer of the
 * pool and the host spins on it (for up to 2 ms, then it blocks in
 * hipStreamSynchronize); the profiled variants, nms_f32_static and calls
 * past the pool copy the control block back and synchronise the stream
 * instead.  Either way, when the call returns *num_kept (a host pointer)
 * is valid and every write of the call to keep_out and the workspace has
 * completed (its last kernel may still be retiring; it writes nothing
 * more).  Inputs must not change until the call returns.
 *
 * Errors.  No exception crosses the ABI.  Every call returns an nms_status;
 * on any status other than NMS_OK, *num_kept (when given) is 0 and keep_out is
 * unspecified.  Device-detected errors (non-finite input, bad offsets) arrive
 * with the same read-back that carries the kept count.
 */
#ifndef GREEDY_NMS_H
#define GREEDY_NMS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nms_status {
    NMS_OK = 0,
    /* A null pointer with n > 0, n < 0, iou_thresh NaN, num_images
     * inconsistent with batch_offsets, or a misaligned boxes pointer. */
    NMS_INVALID_ARG = 1,
    /* workspace_bytes is below what nms_workspace_size reports (one image:
     * below nms_workspace_size_lists, or below nms_workspace_size for an
     * input that needs the dense bitmask). */
    NMS_WORKSPACE_TOO_SMALL = 2,
    /* A NaN score or a non-finite box coordinate (detected on the device). */
    NMS_NONFINITE_INPUT = 3,
    /* batch_offsets not non-decreasing from 0 to n (detected on the device). */
    NMS_BAD_OFFSETS = 4,
    /* n above NMS_MAX_BOXES. */
    NMS_TOO_LARGE = 5,
    /* A HIP runtime call or kernel launch failed. */
    NMS_HIP_ERROR = 6,
    /* Matrix NMS: a box with x1 > x2 or y1 > y2 (detected on the device). */
    NMS_BAD_BOXES = 7
} nms_status;

/* Largest n accepted: one workgroup keeps the removed bitmap (n/8 bytes) in
 * at most 64 KiB of LDS during the sweep. */
#define NMS_MAX_BOXES 512000

/* Stages timed by nms_f32_profiled, in launch order. */
#define NMS_STAGE_SORT 0     /* score keys, stable LSD radix sort, grouping  */
#define NMS_STAGE_GATHER 1   /* sorted box gather + areas + input checks     */
#define NMS_STAGE_MASK 2     /* triangle-tiled IoU suppression bitmask; one  */
                             /* image of 32705 to 262144 boxes: mask and     */
                             /* sweep in one launch (sweep overlaps mask);   */
                             /* the one-launch path for small inputs: the    */
                             /* whole call, timed here                       */
#define NMS_STAGE_SWEEP 3    /* greedy sweep over the mask (+ compaction);   */
                             /* after the fused launch, only its completion  */
                             /* check (or the sweep, if a tile's list of     */
                             /* nonzero words overflowed)                    */
#define NMS_STAGE_COMPACT 4  /* score-order compaction (grouped input only)  */
#define NMS_NUM_STAGES 5

/*
 * nms_workspace_size -- device workspace needed by nms_f32 for n boxes.
 *   n            number of boxes (0 <= n <= NMS_MAX_BOXES)
 *   num_images   number of images in batch_offsets (0 or 1 when there are
 *                none); has_classes: nonzero when class_ids will be given.
 *   *bytes       receives the size; it is a bound computed from n alone
 *                (dominated by the n * ceil(n/64) * 8-byte suppression
 *                bitmask), so no device synchronisation is needed.
 * Returns NMS_OK, NMS_INVALID_ARG (bytes NULL, n < 0) or NMS_TOO_LARGE.
 * Why a bound from n alone: sizing a buffer from the data costs a device
 * round trip before the work can start ("LeetCUDA 12-histogram", its binding
 * section: the max() read back to size the histogram is a forced device
 * synchronisation, which a caller-chosen size avoids).  Our reading: the
 * caller sizes the workspace once from n and reuses it.
 */
nms_status nms_workspace_size(int64_t n, int64_t num_images, int has_classes, size_t *bytes);

/*
 * nms_workspace_size_lists -- a smaller workspace for one image of n boxes:
 * everything but the dense suppression bitmask: about 530 bytes per box,
 * most of it the lists of nonzero mask words (24 KiB per 64 boxes), against
 * n * ceil(n/64) * 8 more bytes for the bitmask (35 MB instead of 572 MB at
 * 65,536 boxes, 273 MB instead of 33 GB at 512,000).
 *   n       number of boxes (0 <= n <= NMS_MAX_BOXES); *bytes receives it.
 * Returns NMS_OK, NMS_INVALID_ARG (bytes NULL, n < 0) or NMS_TOO_LARGE.
 * For one image nms_f32 never writes the dense bitmask unless it must: the
 * sweep reads only the lists of nonzero words of each 64-row tile ("LeetCUDA
 * 14-nms", measured results: the blocked bitmask its authors name as the
 * next step to cut the mask's memory).  A tile with more nonzero words than
 * its list holds (2048: each of its boxes overlapping boxes in 32 or more
 * other tiles on average) needs the dense rows; nms_f32 then runs the call
 * again with them if its workspace holds nms_workspace_size() bytes, and
 * otherwise returns NMS_WORKSPACE_TOO_SMALL (nothing else changes; call
 * again with the larger workspace).  Grouped input always needs
 * nms_workspace_size() bytes.
 */
nms_status nms_workspace_size_lists(int64_t n, size_t *bytes);

/*
 * nms_f32 -- greedy IoU NMS (see the file comment for the exact result).
 *   boxes          device, n*4 floats, row k = (x1, y1, x2, y2) of box k;
 *                  16-byte aligned.
 *   scores         device, n floats.
 *   n              number of boxes; n = 0 returns NMS_OK with *num_kept = 0.
 *   iou_thresh     float32 threshold; any value but NaN (values < 0 remove
 *                  every later box of a group with a defined IoU).
 *   class_ids      device, n int32 class ids, or NULL (one class).
 *   batch_offsets  device, num_images+1 int64 offsets; image m holds boxes
 *                  [off[m], off[m+1]).  NULL = one image (num_images 0 or 1).
 *   keep_out       device, capacity n int64: receives the kept input indices
 *                  in descending score order (ties: ascending index).
 *   num_kept       host: receives the number of kept boxes.
 *   workspace      device scratch of at least nms_workspace_size() bytes
 *                  (one image: nms_workspace_size_lists() bytes will do
 *                  unless the input is dense, see there), 256-byte aligned;
 *                  its contents on entry do not matter.
 *   stream         hipStream_t or NULL.
 * Sorting follows "LeetCUDA 14-nms" step 1 (stable, descending); the
 * bitmask layout follows its Phase 1 (bit k of word w of row i means sorted
 * box 64w + k; only boxes after row i vote); the sweep follows its Phase 2
 * (removed bitmap in on-chip memory, kept rows ORed in in score order); the
 * map-back follows its host section.
 */
nms_status nms_f32(const float *boxes, const float *scores, int64_t n, float iou_thresh,
                   const int32_t *class_ids, const int64_t *batch_offsets, int64_t num_images,
                   int64_t *keep_out, int64_t *num_kept, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Largest n nms_f32_static accepts, and the size of its static scratch. */
#define NMS_STATIC_MAX_BOXES 16384
#define NMS_STATIC_SCRATCH_BYTES (48u << 20)

/*
 * nms_f32_static -- nms_f32 without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It runs the same kernels as
 * nms_f32 on a scratch array that the library holds in its code object: a
 * file-scope device array of NMS_STATIC_SCRATCH_BYTES, one per device the
 * library runs on, allocated by the HIP runtime when the library's code is
 * loaded on that device and held until the process ends.  The call itself
 * allocates nothing: no hipMalloc, no hipHostMalloc (the kept count is
 * copied into the caller's stack frame), no events.
 *   boxes, scores, n, iou_thresh, class_ids, batch_offsets, num_images,
 *   keep_out, num_kept, stream   as for nms_f32.
 * Returns as nms_f32, and NMS_TOO_LARGE for n > NMS_STATIC_MAX_BOXES.
 * Every call on one device shares that device's scratch, which keeps the
 * last call's contents (the kernels need no particular contents on entry):
 * calls that overlap on one device -- from two host threads, or on two
 * streams -- race and must be serialised by the caller.
 */
nms_status nms_f32_static(const float *boxes, const float *scores, int64_t n, float iou_thresh,
                          const int32_t *class_ids, const int64_t *batch_offsets,
                          int64_t num_images, int64_t *keep_out, int64_t *num_kept,
                          void *stream);

/* nms_f32_ex flags. */
#define NMS_FLAG_ONE_LAUNCH 1    /* one image of 1 to 4096 boxes: the whole  */
                                 /* call in a single launch                  */
#define NMS_FLAG_PASS_SORT 2     /* the radix sort as one launch per pass,   */
                                 /* as for inputs above 131072 boxes         */
#define NMS_FLAG_RADIX_SORT 4    /* one image: the radix sort in one launch  */
                                 /* instead of the sample sort               */

/*
 * nms_f32_ex -- nms_f32 with launch-plan flags; flags 0 is nms_f32.
 *   flags   0, or any of NMS_FLAG_ONE_LAUNCH, NMS_FLAG_PASS_SORT and
 *           NMS_FLAG_RADIX_SORT (other bits: NMS_INVALID_ARG).
 * NMS_FLAG_ONE_LAUNCH: one image of 1 to 4096 boxes runs sort, mask, sweep
 * and output in one launch, against the fixed per-launch cost that the
 * "LeetCUDA 14-nms" page (measured results) blames for its losses at 1024
 * and 2048 boxes.  Its workgroups hand over through device memory (a
 * bounded wait on the sort's workgroups, then per-row-tile counters as in
 * the fused launch); if a wait gives up, or a row tile's list of nonzero
 * mask words overflows, the call runs nms_f32's launches instead.  The
 * result is identical either way.  Other inputs ignore the flag.  Our
 * measurement: on MI355X a dependent launch on the same stream costs less
 * than those hand-overs (the three launches of a 1024-box call span 17 us
 * of GPU time, the one launch 25 us), so nms_f32 does not take it.
 * NMS_FLAG_PASS_SORT: grouped input, and one image of more than 16384 boxes,
 * is sorted with one launch per radix pass, the form inputs of more than
 * 131072 boxes always take, instead of by a team of workgroups that stay
 * resident through every pass (one launch).  The result is identical; the
 * flag exists to compare the two (our reading: the pages fix the sort's
 * result, a stable descending order, not its form).
 * NMS_FLAG_RADIX_SORT: one image of 16385 to 131072 boxes, which nms_f32
 * sorts by sample sort in one launch (256 buckets between sampled
 * splitters, each sorted in LDS by one workgroup; a call whose buckets
 * outgrow the LDS runs again with the radix passes), is sorted by the team's
 * radix passes instead.  Same result; the flag exists to compare the two.
 * Other arguments and returns as for nms_f32.
 */
nms_status nms_f32_ex(const float *boxes, const float *scores, int64_t n, float iou_thresh,
                      const int32_t *class_ids, const int64_t *batch_offsets, int64_t num_images,
                      int64_t *keep_out, int64_t *num_kept, void *workspace,
                      size_t workspace_bytes, void *stream, int flags);

/* nms_f32_profiled flags. */
#define NMS_PROFILE_NO_FUSION 1  /* run the mask and the sweep as separate */
                                 /* launches (to time the mask kernel alone) */
#define NMS_PROFILE_ONE_LAUNCH 2 /* as NMS_FLAG_ONE_LAUNCH (timed as the    */
                                 /* mask stage)                              */
#define NMS_PROFILE_PASS_SORT 4  /* as NMS_FLAG_PASS_SORT                    */
#define NMS_PROFILE_RADIX_SORT 8 /* as NMS_FLAG_RADIX_SORT                   */

/*
 * nms_f32_profiled -- nms_f32 with HIP events recorded on `stream` around
 * each stage.  stage_ms (host, NMS_NUM_STAGES floats) receives each stage's
 * elapsed GPU time in milliseconds (0 for a stage that did not run).  flags:
 * 0, NMS_PROFILE_NO_FUSION or NMS_PROFILE_ONE_LAUNCH, with any of
 * NMS_PROFILE_PASS_SORT and NMS_PROFILE_RADIX_SORT (other bits, or the
 * first two together: NMS_INVALID_ARG).  The result is identical to nms_f32's either way.
 */
nms_status nms_f32_profiled(const float *boxes, const float *scores, int64_t n,
                            float iou_thresh, const int32_t *class_ids,
                            const int64_t *batch_offsets, int64_t num_images,
                            int64_t *keep_out, int64_t *num_kept, void *workspace,
                            size_t workspace_bytes, void *stream, float *stage_ms,
                            int flags);

/* Human-readable name of a status ("NMS_OK", ...); never NULL; the
 * returned string is static.  Our reading: the pages' bindings raise
 * exceptions on bad arguments (the device and dtype checks of "LeetCUDA
 * 12-histogram"'s binding section), which cannot cross a C ABI, so every
 * failure is a status code with a name. */
const char *nms_status_string(nms_status status);

/* ---- test-only exports: copy out one stage's intermediate result ---- */

/*
 * nms_debug_order -- run the sort stage only ("LeetCUDA 14-nms", algorithm
 * step 1: a stable descending sort, equal scores in input order; the order is
 * what bug 3's map-back needs).
 *   order_out        device, n int32: input index at each sorted position
 *                    (grouped input: ascending image, then class, then
 *                    descending score, then ascending index).
 *   score_order_out  device, n int32 or NULL: the plain score order
 *                    (descending score, ascending index).
 * Other arguments as for nms_f32; returns as nms_f32 (NMS_NONFINITE_INPUT
 * for a NaN score, with order_out still a permutation).
 */
nms_status nms_debug_order(const float *scores, int64_t n, const int32_t *class_ids,
                           const int64_t *batch_offsets, int64_t num_images,
                           int32_t *order_out, int32_t *score_order_out, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * nms_debug_mask -- run sort, gather and the IoU-mask stage, then expand the
 * mask into a dense row-major array.  The layout is the suppression bitmask
 * of "LeetCUDA 14-nms", Phase 1 (its alignment rule 2: bit k of word w in
 * every row stands for sorted box w * width + k, and boxes at or before the
 * row vote 0), with 64-bit words instead of the page's 32-bit ones.
 *   mask_out   device, n * ceil(n/64) uint64, row stride ceil(n/64) words:
 *              word c of row p (sorted position p) has bit l set iff box
 *              q = 64c + l satisfies p < q < n, q in p's group and
 *              IoU > iou_thresh.  Words the kernel never computes (below
 *              the diagonal tile, beyond the group's last tile) read 0.
 *   order_out  device, n int32 or NULL: the sorted order the rows refer to.
 * Other arguments and returns as for nms_f32.
 */
nms_status nms_debug_mask(const float *boxes, const float *scores, int64_t n,
                          float iou_thresh, const int32_t *class_ids,
                          const int64_t *batch_offsets, int64_t num_images,
                          uint64_t *mask_out, int32_t *order_out, void *workspace,
                          size_t workspace_bytes, void *stream);

/* nms_debug_plan fields. */
#define NMS_PLAN_MASK_QSHIFT 0   /* log2 of the row groups a mask item of the   */
                                 /* separate mask launch is split into (0: the  */
                                 /* sign-test form of the overlap question)     */
#define NMS_PLAN_FUSED 1         /* 1: nms_f32 runs mask and sweep in one launch */
#define NMS_PLAN_FUSED_QSHIFT 2  /* the fused launch's split, -1 if not fused   */
#define NMS_PLAN_RANK_SORT 3     /* 1: the one-launch ranking sort, 0: radix    */
#define NMS_PLAN_SMALL 4         /* 1: the input may take the one-launch path */
                                 /* (one image of 1 to 4096 boxes)             */
#define NMS_PLAN_TEAM_SORT 5     /* 1: the radix sort runs in one launch (a team */
                                 /* of resident workgroups), 0: one launch per  */
                                 /* pass (or the ranking sort)                  */
#define NMS_PLAN_SAMPLE_SORT 6   /* 1: one image sorted by sample sort in one   */
                                 /* launch (before any fallback to the radix)   */
#define NMS_PLAN_FIELDS 8

/*
 * nms_debug_plan -- the launch plan nms_f32 and nms_debug_mask take for n
 * boxes on the current device, without running anything.
 *   plan   host, NMS_PLAN_FIELDS int32: the fields above (unused ones -1;
 *          all -1 for n = 0).
 * Returns NMS_OK, NMS_INVALID_ARG (plan NULL, n < 0, num_images < 0) or
 * NMS_TOO_LARGE.  Our reading: the pages time whole calls only; the plan is
 * exported so that tests can show which kernel form produced a result.
 */
nms_status nms_debug_plan(int64_t n, int64_t num_images, int has_classes, int32_t *plan);

/*
 * nms_debug_decide -- the IoU-mask kernel's threshold test alone: the strict
 * "IoU > threshold" of "LeetCUDA 14-nms" (introduction) on given
 * intersection and union values, decided as the mask kernel decides it (its
 * division-free form is this library's own and must agree with the float32
 * quotient bit for bit, which this export lets a test check).
 *   inter, uni  device, count floats each: an intersection and a union value.
 *   out         device, count bytes: 1 iff the test "inter / uni > t" holds
 *               as the mask kernel decides it.
 *   all_positive_areas  nonzero selects the division-free test the mask
 *               kernel uses when every box has a finite positive area (it
 *               presumes 0 <= inter <= union, union > 0); zero selects the
 *               literal float32 division.
 */
nms_status nms_debug_decide(const float *inter, const float *uni, int64_t count,
                            float iou_thresh, int all_positive_areas, uint8_t *out,
                            void *stream);

/* ------------------------------------------------------------------------
 * Matrix NMS (Gaussian decay), "Fastest Matrix NMS in the West (Part 2)":
 * "What do we need to compute?" and optimisation 4.
 *
 * With the boxes in descending score order (stable, as for nms_f32), the
 * overlap of a father p (earlier) and a child q (later) is the float32 IoU
 * expression above (0/0, two empty boxes, counted as 0); omax[q] is the
 * largest overlap of q with any of its fathers (0 for the first box).  Box q
 * is dropped iff its score is below score_thresh, or some father p gives
 *     exp((omax[p]^2 - O[p][q]^2) / sigma) * score_q  <  score_thresh
 * evaluated in binary64 from the float32 overlaps (the page's
 * s'_j = s_j min_i d_ij < t, with d_ij = exp((O_max,i^2 - O_ij^2) / sigma);
 * the page hard-codes sigma = 0.5).  Every other box is kept; the result is
 * the kept input indices, int64, in descending score order.  Boxes must have
 * x1 <= x2 and y1 <= y2.
 * ------------------------------------------------------------------------ */

/* Stages timed by nms_matrix_f32_profiled. */
#define NMS_MATRIX_STAGE_SORT 0     /* stable sort, gather, scores and checks */
#define NMS_MATRIX_STAGE_OVERLAP 1  /* largest overlap of each box with a father */
#define NMS_MATRIX_STAGE_DECAY 2    /* decay test, kept bitmap, compaction */
#define NMS_MATRIX_NUM_STAGES 3

/*
 * nms_matrix_workspace_size -- device workspace needed by nms_matrix_f32 for
 * n boxes (linear in n: no pairwise matrix is stored).  Returns NMS_OK,
 * NMS_INVALID_ARG (bytes NULL, n < 0) or NMS_TOO_LARGE.
 */
nms_status nms_matrix_workspace_size(int64_t n, size_t *bytes);

/*
 * nms_matrix_f32 -- Matrix NMS as described above.
 *   boxes, scores, n, keep_out, num_kept, workspace, stream  as for nms_f32
 *                  (workspace of at least nms_matrix_workspace_size() bytes).
 *   score_thresh   float32 threshold t on the decayed score; any value but
 *                  NaN.
 *   sigma          Gaussian decay width; finite and > 0 (0.5 on the page).
 * Returns NMS_OK, NMS_INVALID_ARG, NMS_WORKSPACE_TOO_SMALL, NMS_TOO_LARGE,
 * NMS_NONFINITE_INPUT, NMS_BAD_BOXES or NMS_HIP_ERROR.
 */
nms_status nms_matrix_f32(const float *boxes, const float *scores, int64_t n, float score_thresh,
                          double sigma, int64_t *keep_out, int64_t *num_kept, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * nms_matrix_f32_profiled -- nms_matrix_f32 with HIP events on the launch
 * stream around each stage; stage_ms (host, NMS_MATRIX_NUM_STAGES floats)
 * receives the stage times in milliseconds.
 */
nms_status nms_matrix_f32_profiled(const float *boxes, const float *scores, int64_t n,
                                   float score_thresh, double sigma, int64_t *keep_out,
                                   int64_t *num_kept, void *workspace, size_t workspace_bytes,
                                   void *stream, float *stage_ms);

#ifdef __cplusplus
}
#endif

#endif /* GREEDY_NMS_H */
