"""Matrix NMS on the GPU (through the C ABI) against the CPU oracle.

Kept indices must equal the C oracle's element by element.  The decay test
is decided in binary64 on both sides; the library evaluates the literal
exp() expression for every pair within 1e-9 (sigma + 1) of its bound, so the
two can only differ where the oracle itself counts a candidate within a
relative 1e-9 of the threshold (its borderline count), which every input
here is checked to avoid."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "matrix")


def gpu_matrix(boxes, scores, t, sigma=0.5, workspace=None):
    import greedy_iou_nms_amd as g
    dev = device()
    keep = g.matrix_nms(to_dev(np.asarray(boxes, np.float32).reshape(-1, 4), dev),
                        to_dev(np.asarray(scores, np.float32), dev), t, sigma,
                        workspace=workspace)
    return keep.cpu().numpy()


def _check(boxes, scores, t, sigma=0.5, label=""):
    note("matrix %s n=%d t=%r sigma=%r" % (label, len(scores), t, sigma))
    want, border = oracle.c_matrix_nms(boxes, scores, t, sigma, return_borderline=True)
    assert border == 0, "input too close to the threshold for an exact comparison"
    got = gpu_matrix(boxes, scores, t, sigma)
    assert got.dtype == np.int64
    if not np.array_equal(got, want):
        raise AssertionError("%s: %d kept vs oracle %d" % (label, got.size, want.size))


def _golden():
    out = []
    for name in sorted(os.listdir(GOLDEN)):
        d = json.load(open(os.path.join(GOLDEN, name)))
        for k, c in enumerate(d["cases"]):
            out.append(("%s[%d]" % (name[:-5], k), d["boxes"], d["scores"],
                        c["score_threshold"], c.get("sigma", d.get("sigma", 0.5)),
                        c["expected_keep"]))
    return out


GOLDEN_CASES = _golden()


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=[c[0] for c in GOLDEN_CASES])
def test_golden_fixtures(case):
    name, boxes, scores, t, sigma, want = case
    note("matrix golden " + name)
    np.testing.assert_array_equal(gpu_matrix(boxes, scores, t, sigma), want)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 200, 1000, 4097, 8193])
@pytest.mark.parametrize("t,sigma", [(0.1, 0.5), (0.4, 2.0), (0.05, 0.1)])
def test_random_sizes(n, t, sigma):
    w = workloads.random_small(7000 + n, n, canvas=3.0 * np.sqrt(n) + 30)
    _check(w.boxes, w.scores, t, sigma, "random")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_configs(cfg):
    w = workloads.config(cfg, 0)
    _check(w.boxes, w.scores, 0.1, 0.5, w.name)


def test_large_mixed_prefix():
    # the first 12000 boxes of the 65536-box workload (uniform half), plus
    # 4000 of its clustered half
    w = workloads.config(5, 0)
    idx = np.concatenate([np.arange(12000), np.arange(40000, 44000)])
    _check(w.boxes[idx], w.scores[idx], 0.2, 0.5, "large_mixed subset")


def test_full_size_workload():
    # the 65536-box workload the benchmark times, whole: the sort takes the
    # one-launch team form there (the oracle needs tens of seconds)
    w = workloads.config(5, 0)
    _check(w.boxes, w.scores, 0.1, 0.5, "large_mixed full")


def test_ties_and_empty_boxes():
    w = workloads.random_small(91, 3000, canvas=150.0, score_levels=8)
    b = w.boxes.copy()
    b[::13, 2] = b[::13, 0]      # zero width: 0/0 overlaps with other empty boxes
    b[::17, 3] = b[::17, 1]
    _check(b, w.scores, 0.1, 0.5, "ties+empty")


def test_identical_boxes():
    n = 5000
    boxes = np.tile(np.float32([[10, 10, 50, 40]]), (n, 1))
    scores = np.linspace(1.0, 0.05, n).astype(np.float32)
    _check(boxes, scores, 0.1, 0.5, "identical")


def test_signed_scores_and_thresholds():
    # scores below zero and thresholds at or below zero take the literal path
    rng = np.random.default_rng(5)
    w = workloads.random_small(92, 700, canvas=120.0)
    scores = rng.uniform(-1.0, 1.0, 700).astype(np.float32)
    for t in (-0.3, 0.0, 0.2):
        _check(w.boxes, scores, t, 0.5, "signed")


@pytest.mark.parametrize("t", [-0.5, -0.9])
def test_negative_scores_dropped_by_fathers_without_overlap(t):
    # A child with t <= s < 0 can be dropped by a father it does not
    # overlap at all (exp(omax^2 / sigma) s falls below t), so those pairs
    # cannot be skipped; half the scores are negative here and the boxes
    # spread enough that most pairs do not overlap.
    rng = np.random.default_rng(93)
    w = workloads.random_small(93, 1500, canvas=400.0)
    scores = rng.uniform(-1.0, 1.0, 1500).astype(np.float32)
    _check(w.boxes, scores, t, 0.5, "negative scores, sparse")


def test_ten_runs_identical():
    import greedy_iou_nms_amd as g
    w = workloads.config(2, 1)
    dev = device()
    b, s = to_dev(w.boxes, dev), to_dev(w.scores, dev)
    note("matrix ten runs")
    first = g.matrix_nms(b, s, 0.1).cpu().numpy()
    for _ in range(9):
        np.testing.assert_array_equal(g.matrix_nms(b, s, 0.1).cpu().numpy(), first)


def test_device_detected_errors():
    import greedy_iou_nms_amd as g
    dev = device()
    boxes = np.float32([[0, 0, 10, 10], [5, 5, 3, 9], [1, 1, 2, 2]])   # x1 > x2 in box 1
    scores = np.float32([0.9, 0.8, 0.7])
    note("matrix errors")
    with pytest.raises(g.NMSError) as e:
        g.matrix_nms(to_dev(boxes, dev), to_dev(scores, dev), 0.1)
    assert e.value.status == "NMS_BAD_BOXES"
    with pytest.raises(g.NMSError) as e:
        g.matrix_nms(to_dev(boxes[[0, 2]], dev), to_dev(np.float32([np.nan, 0.5]), dev), 0.1)
    assert e.value.status == "NMS_NONFINITE_INPUT"
    # a later good call on the same default workspace is unaffected
    np.testing.assert_array_equal(
        gpu_matrix(boxes[[0, 2]], np.float32([0.9, 0.5]), 0.1),
        oracle.c_matrix_nms(boxes[[0, 2]], np.float32([0.9, 0.5]), 0.1))
