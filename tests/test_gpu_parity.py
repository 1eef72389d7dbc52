"""Parity of the HIP path with the CPU oracle, through the C ABI.

Kept indices must equal the oracle's element by element (integer results,
bit-exact), on hand-built fixtures, on every seeded workload, on the grid of
sizes, seeds and thresholds the LeetCUDA page used for its comparison, on
ragged sizes around the 64-box tile, and on grouped input.
"""
import numpy as np
import pytest

import oracle
import workloads
from golden_cases import load_cases
from gpu_util import gpu_nms, note

pytestmark = pytest.mark.gpu

CASES = load_cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_golden_fixtures(case):
    name, boxes, scores, t, cls, offs, expected = case
    note("golden " + name)
    np.testing.assert_array_equal(gpu_nms(boxes, scores, t, cls, offs), expected)


def _check(w, label=None):
    note("parity %s n=%d t=%r" % (label or w.name, w.n, w.iou_threshold))
    got = gpu_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    assert got.dtype == np.int64
    if not np.array_equal(got, want):
        k = int(np.argmax(got[:min(got.size, want.size)] != want[:min(got.size, want.size)]))
        raise AssertionError("%s: %d kept vs oracle %d; first difference at %d"
                             % (w.name, got.size, want.size, k))
    return got


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_configs_match_oracle(cfg, seed):
    w = workloads.config(cfg, seed)
    got = _check(w)
    if w.n <= 8192:
        assert oracle.certify(w.boxes, w.scores, w.iou_threshold, got,
                              w.class_ids, w.batch_offsets) is None


def test_large_config_matches_oracle():
    _check(workloads.config(5, 0))


@pytest.mark.parametrize("n", [10, 100, 1024, 4096, 8192])
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("t", [0.5, 0.7])
def test_leetcuda_comparison_grid(n, seed, t):
    # sizes x 3 seeds x thresholds {0.5, 0.7} with deliberately tied scores
    # ("LeetCUDA 14-nms", measured results)
    rng = np.random.default_rng(1000 + seed)
    canvas = 40.0 * np.sqrt(n)
    x1 = rng.uniform(0, canvas, n)
    y1 = rng.uniform(0, canvas, n)
    wd = rng.uniform(10, 60, n)
    ht = rng.uniform(10, 60, n)
    boxes = np.stack([x1, y1, x1 + wd, y1 + ht], 1).astype(np.float32)
    scores = (rng.integers(0, 32, n) / 32).astype(np.float32)
    w = workloads.Workload("grid", boxes, scores, t)
    _check(w, "grid n=%d seed=%d" % (n, seed))


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 128, 129, 191, 193, 1000, 1023, 1025,
                               4095, 4097])
def test_ragged_sizes(n):
    w = workloads.random_small(n, n, canvas=8.0 * np.sqrt(n) + 20, score_levels=16)
    _check(w)


@pytest.mark.parametrize("seed", range(12))
def test_grouped_random(seed):
    n = [5, 64, 65, 200, 700, 3000][seed % 6]
    w = workloads.random_small(500 + seed, n, canvas=6.0 * np.sqrt(n) + 30,
                               score_levels=[0, 8][seed % 2], classes=[1, 3, 7][seed % 3],
                               images=[0, 2, 5][seed % 3])
    _check(w)


@pytest.mark.parametrize("t", [0.0, -0.5, 1.0, 1e-30, 0.3, 0.45, 0.7, 0.9, 0.5000001,
                               np.nextafter(np.float32(0.5), np.float32(0))])
def test_thresholds(t):
    w = workloads.random_small(77, 777, canvas=150.0, score_levels=8)
    w.iou_threshold = float(t)
    _check(w)


def test_degenerate_boxes_take_the_division_path():
    rng = np.random.default_rng(5)
    n = 300
    w = workloads.random_small(5, n, canvas=60.0, score_levels=4)
    b = w.boxes.copy()
    b[::7, 2] = b[::7, 0]            # zero width
    b[::11, 3] = b[::11, 1] - 3.0    # inverted height
    pts = rng.integers(0, n, 20)
    b[pts, 2:] = b[pts, :2]          # points
    w.boxes = b
    _check(w)


@pytest.mark.parametrize("n", [8192, 8193, 16384, 16385])
def test_sort_boundary_sizes_with_ties(n):
    # around the largest ranking sort and the smallest radix sort, with few
    # score levels so that the stable order decides
    w = workloads.random_small(800 + n, n, canvas=4.0 * np.sqrt(n) + 30, score_levels=8)
    _check(w)


def test_boxes_inverted_in_both_axes_take_the_division_path():
    # x2 < x1 and y2 < y1 give (x2 - x1) * (y2 - y1) > 0, a positive area,
    # but the division-free test clamps coordinates into an ordered extent
    w = workloads.random_small(6, 500, canvas=80.0, score_levels=4)
    b = w.boxes.copy()
    b[::5] = b[::5][:, [2, 3, 0, 1]]
    w.boxes = b
    _check(w)


def test_equal_scores_everywhere_keep_input_order():
    n = 2000
    rng = np.random.default_rng(9)
    w = workloads.random_small(9, n, canvas=300.0)
    w.scores = np.full(n, 0.5, np.float32)
    w.scores[rng.integers(0, n, 50)] = -0.0
    w.scores[rng.integers(0, n, 50)] = 0.0
    _check(w)
