"""GPU paths that the end-to-end parity tests alone do not reach, each
compared with the oracle:

* the sign-test form of the mask's overlap question (taken when there are
  enough work items, from about 12,000 boxes up), word by word against the
  mask's definition;
* grouped input whose group is wider than the per-segment sweep's window,
  which sends grouped input to the one-workgroup sweep;
* the fused launch at 160,005 boxes (two workgroups per CU), against the
  oracle by way of disjoint clusters;
* Matrix NMS at 65,536 boxes.

Bit layout of the mask: "LeetCUDA 14-nms", Phase 1, alignment rule 2 (with
64-bit words).  Group rule: "YOLOv5 post-processing GPU port", section 2.2.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import device, gpu_nms, note, to_dev

pytestmark = pytest.mark.gpu


def _g():
    import greedy_iou_nms_amd as g
    return g


def _clustered(n, seed, canvas, cluster=16, jitter=6.0, edge_ties=True):
    """Clustered boxes (config-2 law at another size) with some coordinates
    shared exactly between boxes (equal edges give exact zero differences)
    and some boxes at the origin (the zero padding columns use that value)."""
    rng = np.random.default_rng(seed)
    k = (n + cluster - 1) // cluster
    centres = rng.uniform(0, canvas, (k, 2))
    base = rng.uniform(30, 90, (k, 2))
    c = np.arange(n) // cluster
    xy = centres[c] + rng.normal(0, jitter, (n, 2))
    wh = base[c] * (1 + rng.normal(0, 0.1, (n, 2)))
    wh = np.maximum(wh, 1.0)
    boxes = np.concatenate([xy - wh / 2, xy + wh / 2], axis=1)
    if edge_ties:
        m = rng.integers(0, n, n // 20)
        src = rng.integers(0, n, n // 20)
        boxes[m, 0] = boxes[src, 2]       # x1 of one box on x2 of another
        boxes[m, 2] = np.maximum(boxes[m, 2], boxes[m, 0] + 1)
        o = rng.integers(0, n, 8)
        boxes[o] = np.array([0.0, 0.0, 40.0, 40.0])[None]
    scores = rng.beta(2, 5, n)
    return workloads.Workload("clustered_%d" % n, boxes.astype(np.float32),
                              scores.astype(np.float32), 0.5)


# 14,000 boxes: sorted by ranking, the float sign test; 16,385 and more:
# radix-sorted, the quantised pre-test
@pytest.mark.parametrize("n,seed", [(14000, 2), (16385, 0), (20011, 1)])
def test_mask_sign_path_matches_definition(n, seed):
    g = _g()
    device()
    plan = g.debug_plan(n)
    assert plan["mask_qshift"] == 0, plan   # the sign-test form
    assert plan["rank_sort"] == (1 if n <= 16384 else 0), plan
    w = _clustered(n, seed, canvas=2000.0 * np.sqrt(n / 8192))
    note("mask sign path n=%d" % n)
    dev = device()
    m, order = g.debug_mask(to_dev(w.boxes, dev), to_dev(w.scores, dev), w.iou_threshold)
    m = m.cpu().numpy().view(np.uint64)
    order = order.cpu().numpy()
    np.testing.assert_array_equal(order, oracle.stable_order(w.scores))
    want = oracle.mask_rows(w.boxes, w.iou_threshold, order)
    assert int(np.count_nonzero(want)) > n // 4   # the test has suppressions to find
    bad = np.argwhere(m != want)
    assert bad.size == 0, "first differing (row, word): %s" % (bad[:5].tolist(),)


@pytest.mark.parametrize("classes", [1, 3])
def test_grouped_input_with_a_band_wider_than_the_segment_window(classes):
    # 40,000 boxes in one image: a group of over 16,384 boxes has a band of
    # more than 256 row tiles, so the grouped call takes the one-workgroup
    # sweep instead of the per-segment one
    n = 40000
    rng = np.random.default_rng(11 + classes)
    w = workloads.random_small(500 + classes, n, canvas=60.0 + n / 8.0)
    cls = np.zeros(n, np.int32) if classes == 1 else \
        np.where(rng.random(n) < 0.8, 0, rng.integers(1, classes, n)).astype(np.int32)
    offs = np.array([0, n], np.int64)
    note("grouped wide band n=%d classes=%d" % (n, classes))
    got = gpu_nms(w.boxes, w.scores, w.iou_threshold, cls, offs)
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, cls, offs)
    np.testing.assert_array_equal(got, want)
    # and two images of 20,000 each, one class
    offs2 = np.array([0, n // 2, n], np.int64)
    got2 = gpu_nms(w.boxes, w.scores, w.iou_threshold, None, offs2)
    np.testing.assert_array_equal(got2, oracle.c_nms(w.boxes, w.scores, w.iou_threshold,
                                                     None, offs2))


def _disjoint_clusters(n, seed, cluster=16, cell=200.0, cols=400):
    """Clusters of overlapping boxes, each inside its own grid cell with room
    to spare, so boxes of different clusters never overlap.  Greedy NMS of
    the whole input is then the union of the clusters' own results in global
    score order, which the oracle computes with every cluster as an image."""
    rng = np.random.default_rng(seed)
    k = (n + cluster - 1) // cluster
    c = np.arange(n) // cluster
    ox = (c % cols) * cell
    oy = (c // cols) * cell
    x1 = ox + rng.uniform(0, 50, n)
    y1 = oy + rng.uniform(0, 50, n)
    w = rng.uniform(20, 60, n)
    h = rng.uniform(20, 60, n)
    boxes = np.stack([x1, y1, x1 + w, y1 + h], axis=1).astype(np.float32)
    scores = rng.random(n).astype(np.float32)
    offs = np.minimum(np.arange(0, k + 1) * cluster, n).astype(np.int64)
    return boxes, scores, offs


def test_fused_two_workgroups_per_cu_against_oracle():
    # 2501 row tiles: the removed bitmap leaves LDS room for two fused
    # workgroups per CU instead of three
    g = _g()
    n = 64 * 2500 + 5
    plan = g.debug_plan(n)
    assert plan["fused"] == 1
    boxes, scores, offs = _disjoint_clusters(n, 17)
    note("fused two workgroups per CU n=%d vs oracle" % n)
    want = oracle.c_nms(boxes, scores, 0.5, None, offs)
    assert 0 < want.size < n
    got = gpu_nms(boxes, scores, 0.5)
    np.testing.assert_array_equal(got, want)


def test_disjoint_cluster_decomposition_on_the_oracle():
    # the decomposition itself, checked where the oracle runs the whole
    # single-image problem in seconds
    boxes, scores, offs = _disjoint_clusters(6000, 18)
    np.testing.assert_array_equal(oracle.c_nms(boxes, scores, 0.5),
                                  oracle.c_nms(boxes, scores, 0.5, None, offs))


def test_matrix_nms_large_mixed_against_oracle():
    g = _g()
    dev = device()
    w = workloads.config(5, 0)
    note("matrix nms n=%d vs oracle" % w.n)
    got = g.matrix_nms(to_dev(w.boxes, dev), to_dev(w.scores, dev), 0.1, 0.5).cpu().numpy()
    want = oracle.c_matrix_nms(w.boxes, w.scores, 0.1, 0.5)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("kind", ["wide_range", "negative_far", "tiny_boxes"])
def test_quantised_pretest_on_extreme_ranges(kind):
    # The pre-test quantises coordinates to 15 bits over the extent of all
    # boxes: a huge extent makes its grid coarse (it then rules out less),
    # never wrong.  Word by word against the definition, and end to end.
    g = _g()
    dev = device()
    n = 20011
    rng = np.random.default_rng({"wide_range": 1, "negative_far": 2, "tiny_boxes": 3}[kind])
    w = _clustered(n, 31, canvas=3000.0, edge_ties=False)
    b = w.boxes.astype(np.float64)
    if kind == "wide_range":
        b[:50] += rng.uniform(-1e7, 1e7, (50, 1))          # a few boxes far out
    elif kind == "negative_far":
        b -= 5e6                                            # large negative coordinates
    else:
        c = b[:, :2] + (b[:, 2:] - b[:, :2]) / 2
        s = rng.uniform(1e-3, 3e-3, (n, 1))
        b = np.concatenate([c / 1000 - s, c / 1000 + s], axis=1)   # tiny boxes, tiny canvas
    w = workloads.Workload(kind, b.astype(np.float32), w.scores, 0.5)
    assert np.all(w.boxes[:, 0] < w.boxes[:, 2]) and np.all(w.boxes[:, 1] < w.boxes[:, 3])
    note("quantised pre-test %s n=%d" % (kind, n))
    m, order = g.debug_mask(to_dev(w.boxes, dev), to_dev(w.scores, dev), w.iou_threshold)
    m = m.cpu().numpy().view(np.uint64)
    order = order.cpu().numpy()
    want = oracle.mask_rows(w.boxes, w.iou_threshold, order)
    bad = np.argwhere(m != want)
    assert bad.size == 0, "first differing (row, word): %s" % (bad[:5].tolist(),)
    np.testing.assert_array_equal(gpu_nms(w.boxes, w.scores, w.iou_threshold),
                                  oracle.c_nms(w.boxes, w.scores, w.iou_threshold))


@pytest.mark.parametrize("seed", [0, 1])
def test_coarse_pretest_cell_boundaries(seed):
    # The coarse pre-test cuts the grid to 7 bits: on an extent of exactly
    # 0 .. 32766 the fine grid step is 1 and a coarse cell is 256 wide.  Box
    # edges sit on and within 2 of the cell edges, boxes touch (x2 of one on
    # x1 of another) and shifted copies overlap across cells, so pairs in the
    # same, adjacent and next-but-one cells all occur.  Word by word against
    # the definition, and end to end.
    g = _g()
    dev = device()
    rng = np.random.default_rng(40 + seed)
    n = 20000
    base = n // 2

    def edge(cells, jit):
        return 256.0 * cells + rng.choice(jit, cells.shape)

    x1 = np.clip(edge(rng.integers(0, 120, base), [-2, -1, -0.5, 0, 0.5, 1, 2]), 0, None)
    y1 = np.clip(edge(rng.integers(0, 120, base), [-2, -1, 0, 1, 2]), 0, None)
    x2 = x1 + edge(rng.integers(1, 3, base), [-2, -1, 0, 1, 2])
    y2 = y1 + edge(rng.integers(1, 3, base), [-2, -1, 0, 1, 2])
    a = np.stack([x1, y1, x2, y2], axis=1)
    src = rng.integers(0, base, n - base)
    b = a[src].copy()
    shift = rng.choice([-260.0, -256.0, -40.0, -1.0, 1.0, 40.0, 256.0, 260.0], (n - base, 2))
    b[:, [0, 2]] += shift[:, :1]
    b[:, [1, 3]] += shift[:, 1:]
    touch = rng.integers(0, n - base, (n - base) // 10)
    b[touch, 0] = a[src[touch], 2]                      # x1 on the source's x2
    b[touch, 2] = b[touch, 0] + 256.0
    boxes = np.concatenate([a, b])
    boxes = np.clip(boxes, 0.0, 32766.0)
    boxes[:, 2] = np.maximum(boxes[:, 2], boxes[:, 0] + 1.0)
    boxes[:, 3] = np.maximum(boxes[:, 3], boxes[:, 1] + 1.0)
    boxes[0] = [0.0, 0.0, 10.0, 10.0]                   # the extent: 0 .. 32766
    boxes[1] = [32756.0, 32756.0, 32766.0, 32766.0]
    boxes = boxes.astype(np.float32)
    scores = rng.random(n).astype(np.float32)
    w = workloads.Workload("coarse_cells_%d" % seed, boxes, scores, 0.3)
    assert g.debug_plan(n)["rank_sort"] == 0            # radix-sorted: the pre-test words exist
    note("coarse pre-test cell boundaries seed=%d" % seed)
    m, order = g.debug_mask(to_dev(w.boxes, dev), to_dev(w.scores, dev), w.iou_threshold)
    m = m.cpu().numpy().view(np.uint64)
    order = order.cpu().numpy()
    want = oracle.mask_rows(w.boxes, w.iou_threshold, order)
    assert int(np.count_nonzero(want)) > n // 10        # overlaps to find
    bad = np.argwhere(m != want)
    assert bad.size == 0, "first differing (row, word): %s" % (bad[:5].tolist(),)
    np.testing.assert_array_equal(gpu_nms(w.boxes, w.scores, w.iou_threshold),
                                  oracle.c_nms(w.boxes, w.scores, w.iou_threshold))
