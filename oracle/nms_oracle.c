/*
 * CPU oracle for greedy IoU non-maximum suppression.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the GPU library against a plain,
 * slow, obviously correct definition.  It shares no code, header or constant
 * with the GPU library.
 *
 * What it computes (the textbook definition, step by step):
 *
 *   1. Validate the inputs (finite coordinates, no NaN score, monotone batch
 *      offsets from 0 to n).
 *   2. Give every box a group = (image from the batch offsets, class id);
 *      a missing part is 0.  Suppression happens only inside a group
 *      (the class check of "YOLOv5 post-processing GPU port", section 2.2).
 *   3. Sort the box indices by score, highest first, with a stable sort, so
 *      equal scores keep ascending input order ("LeetCUDA 14-nms", algorithm
 *      and data flow, step 1; the same page's bug 3 on the torch stable sort;
 *      the Matrix NMS page's PyTorch-extension section sorts with stable=true).
 *   4. removed[] starts all-false (the "zeros, not empty" fix of bug 1 on the
 *      LeetCUDA page).
 *   5. Visit boxes in that order; a box not yet removed is kept, and it
 *      removes every later box of its group whose IoU with it exceeds the
 *      threshold, strictly (the introduction of the LeetCUDA page: keep
 *      greedily by score, delete boxes overlapping a kept box with IoU > t).
 *   6. Return the kept boxes as their ORIGINAL input indices, int64, in the
 *      visiting order (the host-side map-back of bug 3 on the LeetCUDA page).
 *
 * The IoU is one fixed float32 expression, every step one IEEE binary32
 * operation, no fused multiply-add (build with -ffp-contract=off, SSE math):
 *   area  = (x2 - x1) * (y2 - y1)            once per box
 *   w     = max(min(x2i,x2j) - max(x1i,x1j), 0)
 *   h     = max(min(y2i,y2j) - max(y1i,y1j), 0)
 *   inter = w * h
 *   uni   = (area_i + area_j) - inter
 *   iou   = inter / uni                      correctly rounded division
 *   suppress iff iou > t                     t is the float32 threshold
 * None of the pages prints its IoU routine; this expression (no "+1" on the
 * widths, union summed left to right) is the reading this oracle fixes.
 *
 * Status values returned (the oracle's own numbering):
 *   0 ok, 1 invalid argument, 3 non-finite input, 4 bad batch offsets.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_INVALID_ARG 1
#define ORACLE_NONFINITE 3
#define ORACLE_BAD_OFFSETS 4

static float fmax_plain(float a, float b) { return a > b ? a : b; }
static float fmin_plain(float a, float b) { return a < b ? a : b; }

static float box_area(const float *b) {
    float w = b[2] - b[0];
    float h = b[3] - b[1];
    return w * h;
}

/* The float32 IoU of boxes i and j, given their areas. */
static float box_iou(const float *bi, float ai, const float *bj, float aj) {
    float xx1 = fmax_plain(bi[0], bj[0]);
    float yy1 = fmax_plain(bi[1], bj[1]);
    float xx2 = fmin_plain(bi[2], bj[2]);
    float yy2 = fmin_plain(bi[3], bj[3]);
    float w = fmax_plain(xx2 - xx1, 0.0f);
    float h = fmax_plain(yy2 - yy1, 0.0f);
    float inter = w * h;
    float uni = (ai + aj) - inter;
    return inter / uni;
}

/* Stable merge sort of idx[0..n) by score, descending: an element from the
 * right run is taken first only when its score is strictly greater. */
static void stable_sort_desc(int64_t *idx, int64_t *tmp, int64_t n, const float *score) {
    for (int64_t width = 1; width < n; width *= 2) {
        for (int64_t lo = 0; lo < n; lo += 2 * width) {
            int64_t mid = lo + width < n ? lo + width : n;
            int64_t hi = lo + 2 * width < n ? lo + 2 * width : n;
            int64_t a = lo, b = mid, o = lo;
            while (a < mid && b < hi) {
                if (score[idx[b]] > score[idx[a]]) tmp[o++] = idx[b++];
                else tmp[o++] = idx[a++];
            }
            while (a < mid) tmp[o++] = idx[a++];
            while (b < hi) tmp[o++] = idx[b++];
        }
        memcpy(idx, tmp, (size_t)n * sizeof(int64_t));
    }
}

/*
 * oracle_nms: greedy IoU NMS by definition.
 *   boxes[n*4] (x1,y1,x2,y2), scores[n], iou_thresh (float32),
 *   class_ids[n] or NULL, batch_offsets[num_images+1] or NULL,
 *   keep_out[n] receives kept input indices in visiting order,
 *   *num_kept their count.
 *   borderline_out (may be NULL): number of evaluated pairs whose float32 IoU
 *   lies within 1e-6 of the threshold (compared in double).
 */
int oracle_nms(const float *boxes, const float *scores, int64_t n, float iou_thresh,
               const int32_t *class_ids, const int64_t *batch_offsets, int64_t num_images,
               int64_t *keep_out, int64_t *num_kept, int64_t *borderline_out) {
    if (num_kept == NULL || n < 0 || isnan(iou_thresh)) return ORACLE_INVALID_ARG;
    if (n > 0 && (boxes == NULL || scores == NULL || keep_out == NULL)) return ORACLE_INVALID_ARG;
    if (batch_offsets == NULL && num_images > 1) return ORACLE_INVALID_ARG;
    if (batch_offsets != NULL && num_images < 1) return ORACLE_INVALID_ARG;
    *num_kept = 0;
    if (borderline_out) *borderline_out = 0;

    if (batch_offsets != NULL) {
        if (batch_offsets[0] != 0 || batch_offsets[num_images] != n) return ORACLE_BAD_OFFSETS;
        for (int64_t m = 0; m < num_images; ++m)
            if (batch_offsets[m + 1] < batch_offsets[m]) return ORACLE_BAD_OFFSETS;
    }
    for (int64_t k = 0; k < n; ++k) {
        if (isnan(scores[k])) return ORACLE_NONFINITE;
        for (int c = 0; c < 4; ++c)
            if (!isfinite(boxes[4 * k + c])) return ORACLE_NONFINITE;
    }
    if (n == 0) return ORACLE_OK;

    int64_t *image = (int64_t *)calloc((size_t)n, sizeof(int64_t));
    int64_t *order = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    int64_t *tmp = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    float *area = (float *)malloc((size_t)n * sizeof(float));
    unsigned char *removed = (unsigned char *)calloc((size_t)n, 1);
    if (!image || !order || !tmp || !area || !removed) {
        free(image); free(order); free(tmp); free(area); free(removed);
        return ORACLE_INVALID_ARG;
    }
    if (batch_offsets != NULL)
        for (int64_t m = 0; m < num_images; ++m)
            for (int64_t k = batch_offsets[m]; k < batch_offsets[m + 1]; ++k) image[k] = m;
    for (int64_t k = 0; k < n; ++k) {
        order[k] = k;
        area[k] = box_area(boxes + 4 * k);
    }
    stable_sort_desc(order, tmp, n, scores);

    int64_t kept = 0, borderline = 0;
    for (int64_t p = 0; p < n; ++p) {
        int64_t i = order[p];
        if (removed[i]) continue;
        keep_out[kept++] = i;
        for (int64_t q = p + 1; q < n; ++q) {
            int64_t j = order[q];
            if (removed[j]) continue;
            if (image[j] != image[i]) continue;
            if (class_ids != NULL && class_ids[j] != class_ids[i]) continue;
            float iou = box_iou(boxes + 4 * i, area[i], boxes + 4 * j, area[j]);
            if (borderline_out && fabs((double)iou - (double)iou_thresh) <= 1e-6) ++borderline;
            if (iou > iou_thresh) removed[j] = 1;
        }
    }
    *num_kept = kept;
    if (borderline_out) *borderline_out = borderline;
    free(image); free(order); free(tmp); free(area); free(removed);
    return ORACLE_OK;
}

/* The float32 IoU of every pair (a[k], b[k]) of box indices, for tests that
 * pin the expression on hand-computed values. */
void oracle_pair_iou(const float *boxes, const int64_t *a, const int64_t *b, int64_t count,
                     float *iou_out) {
    for (int64_t k = 0; k < count; ++k) {
        const float *bi = boxes + 4 * a[k];
        const float *bj = boxes + 4 * b[k];
        iou_out[k] = box_iou(bi, box_area(bi), bj, box_area(bj));
    }
}

/*
 * oracle_matrix_nms: Matrix NMS with the Gaussian decay, by definition
 * ("Fastest Matrix NMS in the West (Part 2)", "What do we need to compute?"
 * and optimisation 4).
 *
 *   1. Validate: finite coordinates, no NaN score, x1 <= x2 and y1 <= y2 for
 *      every box (so an IoU is 0..1 or 0/0), sigma finite and > 0, the
 *      threshold not NaN.
 *   2. Stable descending score sort, as for greedy NMS (the page's extension
 *      sorts with stable=true).
 *   3. O[p][q] for sorted positions p < q: the float32 IoU expression above of
 *      father p and child q; 0/0 (two empty boxes) counts as overlap 0.
 *   4. omax[q] = the largest O[p][q] over the fathers p < q (0 for q = 0).
 *   5. Box q is dropped iff its score is below the threshold or some father p
 *      gives a candidate decayed score below it:
 *          x    = ((double)omax[p]^2 - (double)O[p][q]^2) / sigma
 *          cand = exp(x) * (double)score
 *          cand < (double)score_thresh
 *      (the page: s'_j = s_j min_i d_ij with d_ij = exp((O_max,i^2 -
 *      O_ij^2)/sigma), and "s'_j < t iff some s_j d_ij < t" for non-negative
 *      scores; for a box with no fathers, or any box whose score is below t,
 *      the decay of the first box -- which never exceeds 1 -- makes the score
 *      alone decide).  The decay is evaluated in binary64, after the float32
 *      IoUs.
 *   6. The kept boxes as original input indices, in sorted order.
 *
 * borderline_out (may be NULL): boxes decided by a candidate within a
 * relative 1e-9 of the threshold, where two exp() implementations could
 * disagree.  Status values as oracle_nms, plus 5 = a box with x1 > x2 or
 * y1 > y2.
 */
#define ORACLE_BAD_BOXES 5

static float overlap_or_zero(const float *bi, float ai, const float *bj, float aj) {
    float o = box_iou(bi, ai, bj, aj);
    return o == o ? o : 0.0f;
}

int oracle_matrix_nms(const float *boxes, const float *scores, int64_t n, float score_thresh,
                      double sigma, int64_t *keep_out, int64_t *num_kept,
                      int64_t *borderline_out) {
    if (num_kept == NULL || n < 0 || isnan(score_thresh) || !isfinite(sigma) || !(sigma > 0.0))
        return ORACLE_INVALID_ARG;
    if (n > 0 && (boxes == NULL || scores == NULL || keep_out == NULL)) return ORACLE_INVALID_ARG;
    *num_kept = 0;
    if (borderline_out) *borderline_out = 0;
    for (int64_t k = 0; k < n; ++k) {
        if (isnan(scores[k])) return ORACLE_NONFINITE;
        for (int c = 0; c < 4; ++c)
            if (!isfinite(boxes[4 * k + c])) return ORACLE_NONFINITE;
    }
    for (int64_t k = 0; k < n; ++k)
        if (boxes[4 * k] > boxes[4 * k + 2] || boxes[4 * k + 1] > boxes[4 * k + 3])
            return ORACLE_BAD_BOXES;
    if (n == 0) return ORACLE_OK;

    int64_t *order = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    int64_t *tmp = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    float *area = (float *)malloc((size_t)n * sizeof(float));
    float *omax = (float *)calloc((size_t)n, sizeof(float));
    if (!order || !tmp || !area || !omax) {
        free(order); free(tmp); free(area); free(omax);
        return ORACLE_INVALID_ARG;
    }
    for (int64_t k = 0; k < n; ++k) {
        order[k] = k;
        area[k] = box_area(boxes + 4 * k);
    }
    stable_sort_desc(order, tmp, n, scores);

    for (int64_t q = 1; q < n; ++q) {
        const int64_t j = order[q];
        float m = 0.0f;
        for (int64_t p = 0; p < q; ++p) {
            const int64_t i = order[p];
            float o = overlap_or_zero(boxes + 4 * i, area[i], boxes + 4 * j, area[j]);
            if (o > m) m = o;
        }
        omax[q] = m;
    }

    const double t = (double)score_thresh;
    int64_t kept = 0, borderline = 0;
    for (int64_t q = 0; q < n; ++q) {
        const int64_t j = order[q];
        const double s = (double)scores[j];
        int drop = s < t;
        for (int64_t p = 0; p < q && !drop; ++p) {
            const int64_t i = order[p];
            float o = overlap_or_zero(boxes + 4 * i, area[i], boxes + 4 * j, area[j]);
            double x = ((double)omax[p] * (double)omax[p] - (double)o * (double)o) / sigma;
            double cand = exp(x) * s;
            if (fabs(cand - t) <= 1e-9 * fabs(t)) ++borderline;
            if (cand < t) drop = 1;
        }
        if (!drop) keep_out[kept++] = j;
    }
    *num_kept = kept;
    if (borderline_out) *borderline_out = borderline;
    free(order); free(tmp); free(area); free(omax);
    return ORACLE_OK;
}
