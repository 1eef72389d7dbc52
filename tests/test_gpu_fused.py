"""The fused launch (IoU mask and sweep together, one image of 512 to 4096
row tiles): its result must equal the separate launches' and the oracle's,
also where it gives up (a row tile with more nonzero mask words than its
list holds) and leaves the work to the plain sweep, and outside the size
range of fusion."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu


def _both(w):
    import greedy_iou_nms_amd as g
    dev = device()
    b = to_dev(np.asarray(w.boxes, np.float32).reshape(-1, 4), dev)
    s = to_dev(np.asarray(w.scores, np.float32), dev)
    fused, st_f = g.nms_profiled(b, s, w.iou_threshold)
    sep, st_s = g.nms_profiled(b, s, w.iou_threshold, fuse=False)
    plain = g.nms(b, s, w.iou_threshold)
    return fused.cpu().numpy(), sep.cpu().numpy(), plain.cpu().numpy(), st_f, st_s


@pytest.mark.parametrize("cfg,seed", [(1, 0), (2, 0), (2, 1), (3, 0), (5, 0), (5, 2)])
def test_fused_equals_separate_and_oracle(cfg, seed):
    w = workloads.config(cfg, seed)
    note("fused vs separate cfg=%d seed=%d" % (cfg, seed))
    fused, sep, plain, _, _ = _both(w)
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold)
    np.testing.assert_array_equal(fused, want)
    np.testing.assert_array_equal(sep, want)
    np.testing.assert_array_equal(plain, want)


@pytest.mark.parametrize("n", [1, 65, 4097, 32704, 32705, 40000 + 37])
def test_fused_ragged_sizes(n):
    # 32704 boxes: 511 row tiles, separate launches; 32705: 512, fused
    w = workloads.random_small(n, n, canvas=60.0 + n / 8.0)
    note("fused ragged n=%d" % n)
    fused, sep, _, _, _ = _both(w)
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold)
    np.testing.assert_array_equal(fused, want)
    np.testing.assert_array_equal(sep, want)


def test_fused_with_two_workgroups_per_cu():
    # 2501 row tiles: the removed bitmap (20 KB) beside the sweep's 42.8 KB
    # of LDS leaves room for two workgroups per CU instead of three, so the
    # fused launch takes its other occupancy and splits its items for it.
    # The oracle comparison at this size is in test_gpu_coverage.py (on
    # disjoint clusters); here the three launch forms must agree on the
    # uniform boxes.
    n = 64 * 2500 + 5
    w = workloads.random_small(4242, n, canvas=60.0 + n / 8.0)
    note("fused two workgroups per CU n=%d" % n)
    fused, sep, plain, _, _ = _both(w)
    assert fused.size > 0
    np.testing.assert_array_equal(fused, sep)
    np.testing.assert_array_equal(plain, sep)


def test_fused_size_with_inverted_boxes():
    # a few boxes with x2 < x1 and y2 < y1 (positive area) send the whole
    # call to the literal division test, at a size the fused launch takes
    n = 40000 + 37
    w = workloads.random_small(n, n, canvas=60.0 + n / 8.0)
    b = w.boxes.copy()
    b[::997] = b[::997][:, [2, 3, 0, 1]]
    w.boxes = b
    note("fused inverted n=%d" % n)
    fused, sep, _, _, _ = _both(w)
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold)
    np.testing.assert_array_equal(fused, want)
    np.testing.assert_array_equal(sep, want)


def test_fused_gives_up_on_list_overflow():
    # copies of one box: every row of a tile suppresses all later boxes,
    # 64 rows x hundreds of nonzero words is more than a tile's list holds,
    # so the fused sweep stops and the plain sweep produces the result
    n = 40000
    boxes = np.tile(np.array([[10.0, 10.0, 50.0, 50.0]], np.float32), (n, 1))
    scores = np.linspace(1.0, 0.1, n).astype(np.float32)
    w = workloads.Workload("identical", boxes, scores, 0.5)
    note("fused overflow n=%d" % n)
    fused, sep, _, _, _ = _both(w)
    np.testing.assert_array_equal(fused, [0])
    np.testing.assert_array_equal(sep, [0])


def test_fused_ten_runs_identical():
    w = workloads.config(5, 1)
    note("fused determinism cfg=5 seed=1")
    import greedy_iou_nms_amd as g
    dev = device()
    b = to_dev(w.boxes, dev)
    s = to_dev(w.scores, dev)
    first = g.nms(b, s, w.iou_threshold).cpu().numpy()
    np.testing.assert_array_equal(first, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))
    for _ in range(9):
        assert np.array_equal(first, g.nms(b, s, w.iou_threshold).cpu().numpy())


def _pairs_on_a_grid(n, seed):
    """Boxes 2c and 2c+1 are identical and sit alone in grid cell c (10 x 10
    boxes on a 20-pixel grid, so different cells never overlap).  Greedy NMS
    keeps, of each pair, the box with the higher score (the lower index on
    equal scores), and returns the kept boxes in stable score order."""
    rng = np.random.default_rng(seed)
    cell = np.arange(n) // 2
    x = (cell % 1024) * 20.0
    y = (cell // 1024) * 20.0
    boxes = np.stack([x, y, x + 10.0, y + 10.0], axis=1).astype(np.float32)
    scores = rng.integers(0, 1000, n).astype(np.float32) / 1000.0
    first = np.arange(0, n, 2)
    second = np.minimum(first + 1, n - 1)
    winner = np.where(scores[second] > scores[first], second, first)
    order = np.lexsort((winner, -scores[winner]))
    return boxes, scores, winner[order]


def test_pairs_closed_form_fused():
    n = 65536 + 40
    boxes, scores, want = _pairs_on_a_grid(n, 3)
    w = workloads.Workload("pairs", boxes, scores, 0.5)
    note("pairs closed form n=%d" % n)
    fused, sep, _, _, _ = _both(w)
    np.testing.assert_array_equal(fused, want)
    np.testing.assert_array_equal(sep, want)


def test_above_fusion_limit_uses_separate_launches():
    # 4097 row tiles: one more than the fused launch takes
    n = 64 * 4096 + 64
    boxes, scores, want = _pairs_on_a_grid(n, 4)
    w = workloads.Workload("pairs", boxes, scores, 0.5)
    note("above fusion limit n=%d" % n)
    fused, sep, _, _, _ = _both(w)
    np.testing.assert_array_equal(fused, want)
    np.testing.assert_array_equal(sep, want)


def test_largest_accepted_size():
    # NMS_MAX_BOXES = 512000: 8000 row tiles, the plain sweep's removed
    # bitmap at its largest (64 KB of LDS beside the staging ring)
    n = 512000
    boxes, scores, want = _pairs_on_a_grid(n, 5)
    w = workloads.Workload("pairs", boxes, scores, 0.5)
    note("largest size n=%d" % n)
    import greedy_iou_nms_amd as g
    dev = device()
    got = g.nms(to_dev(boxes, dev), to_dev(scores, dev), 0.5).cpu().numpy()
    np.testing.assert_array_equal(got, want)
    del w
