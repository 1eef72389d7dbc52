"""Pins for the CPU oracle (no GPU needed).

The oracle is checked against facts fixed outside itself: hand-computed
fixtures under tests/golden/ (each with its citation), closed forms that hold
at any size, brute-force enumeration on tiny inputs, the independent numpy
implementation and the certificate checker.  ``test_planted_mistakes`` shows
that each plausible slip in the C oracle fails at least one of these pins.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from golden_cases import load_cases, load_raw

CASES = load_cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_golden_c_oracle(case):
    name, boxes, scores, t, cls, offs, expected = case
    got = oracle.c_nms(boxes, scores, t, cls, offs)
    assert got.dtype == np.int64
    np.testing.assert_array_equal(got, expected)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_golden_numpy_oracle(case):
    name, boxes, scores, t, cls, offs, expected = case
    np.testing.assert_array_equal(oracle.np_nms(boxes, scores, t, cls, offs), expected)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_golden_certificate(case):
    name, boxes, scores, t, cls, offs, expected = case
    assert oracle.certify(boxes, scores, t, expected, cls, offs) is None
    if boxes.shape[0] <= 12:
        np.testing.assert_array_equal(oracle.brute_force(boxes, scores, t, cls, offs), expected)


def test_chain_is_not_fast_nms():
    d = load_raw("chain3")
    got = oracle.c_nms(np.float32(d["boxes"]), np.float32(d["scores"]), d["iou_threshold"])
    assert got.tolist() == d["expected_keep"] != d["fast_nms_keep"]


# IoU values worked out by hand; every one is the float32 rounding of the
# exact rational because each intermediate step is exact for these inputs.
IOU_PAIRS = [
    ([0, 0, 10, 10], [5, 0, 15, 10], 50 / 150),      # half overlap: 1/3
    ([0, 0, 10, 10], [0, 0, 10, 5], 0.5),            # nested half box
    ([0, 0, 4, 4], [2, 2, 6, 6], 4 / 28),            # corner overlap: 1/7
    ([0, 0, 10, 10], [2, 2, 4, 4], 4 / 100),         # contained small box
    ([0, 0, 10, 10], [10, 0, 20, 10], 0.0),          # touching edge
    ([0, 0, 10, 10], [30, 30, 40, 40], 0.0),         # disjoint
    ([0, 0, 10, 10], [0, 0, 10, 10], 1.0),           # identical
    ([0, 0, 1, 1], [0.5, 0, 1.5, 1], 0.5 / 1.5),     # half-unit shift
    ([0, 0, 2, 3], [1, 1, 3, 4], 2 / 10),            # 1x2 overlap of 6+6
    ([0, 0, 10, 10], [20, 0, 30, 10], 0.0),          # apart in x only
    ([0, 0, 10, 10], [20, 20, 30, 30], 0.0),         # apart in x and y
]


def test_iou_expression_values():
    boxes = np.float32([p for a, b, _ in IOU_PAIRS for p in (a, b)])
    a = np.arange(0, 2 * len(IOU_PAIRS), 2)
    got = oracle.c_pair_iou(boxes, a, a + 1)
    want = np.float32([v for _, _, v in IOU_PAIRS])
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(oracle.np_iou_pairs(boxes, a, a + 1), want)
    # symmetric in its operands, bit for bit
    np.testing.assert_array_equal(oracle.c_pair_iou(boxes, a + 1, a), want)


def test_iou_float32_union_rounding():
    d = load_raw("fp32_union_rounding")
    boxes = np.float32(d["boxes"])
    got = oracle.c_pair_iou(boxes, np.array([0]), np.array([1]))[0]
    assert got == np.float32(d["expected_iou_f32"])
    assert got > np.float32(0.5)
    # exact arithmetic would give exactly one half
    assert 5592407 / (2 * 5592407) == 0.5


def _random_boxes(rng, n, canvas=100.0, lo=2.0, hi=30.0):
    x1 = rng.uniform(0, canvas, n)
    y1 = rng.uniform(0, canvas, n)
    w = rng.uniform(lo, hi, n)
    h = rng.uniform(lo, hi, n)
    return np.stack([x1, y1, x1 + w, y1 + h], 1).astype(np.float32)


def test_closed_form_threshold_one_keeps_all_in_stable_order():
    # IoU never exceeds 1 for positive-area boxes, so t = 1 removes nothing
    rng = np.random.default_rng(11)
    for n in (1, 7, 64, 65, 300):
        boxes = _random_boxes(rng, n, canvas=20.0)
        scores = (rng.integers(0, 5, n) / 4).astype(np.float32)
        want = np.argsort(-scores, kind="stable")
        np.testing.assert_array_equal(oracle.c_nms(boxes, scores, 1.0), want)


def test_closed_form_negative_threshold_keeps_one_per_group():
    # every IoU of positive-area boxes is >= 0 > t: each group keeps its first box
    rng = np.random.default_rng(12)
    for n in (1, 10, 257):
        boxes = _random_boxes(rng, n)
        scores = (rng.integers(0, 7, n) / 8).astype(np.float32)
        cls = rng.integers(0, 5, n).astype(np.int32)
        cuts = np.sort(rng.integers(0, n + 1, 2))
        offs = np.array([0, cuts[0], cuts[1], n], dtype=np.int64)
        img = np.repeat(np.arange(3), np.diff(offs))
        seen, want = set(), []
        for i in np.argsort(-scores, kind="stable"):
            g = (img[i], cls[i])
            if g not in seen:
                seen.add(g)
                want.append(i)
        np.testing.assert_array_equal(oracle.c_nms(boxes, scores, -0.25, cls, offs), want)


def test_closed_form_disjoint_grid_keeps_everything():
    rng = np.random.default_rng(13)
    k = 17
    gx, gy = np.meshgrid(np.arange(k) * 10.0, np.arange(k) * 10.0)
    x1, y1 = gx.ravel(), gy.ravel()
    boxes = np.stack([x1, y1, x1 + 9, y1 + 9], 1).astype(np.float32)
    scores = rng.random(k * k).astype(np.float32)
    np.testing.assert_array_equal(oracle.c_nms(boxes, scores, 0.0),
                                  np.argsort(-scores, kind="stable"))


def test_closed_form_identical_boxes_keep_one():
    rng = np.random.default_rng(14)
    for n in (2, 3, 100, 1000):
        boxes = np.tile(np.float32([[3, 4, 9, 12]]), (n, 1))
        scores = (rng.integers(0, 3, n) / 2).astype(np.float32)
        want = [int(np.argsort(-scores, kind="stable")[0])]
        assert oracle.c_nms(boxes, scores, 0.5).tolist() == want


def test_brute_force_agrees_on_tiny_random_inputs():
    rng = np.random.default_rng(15)
    for trial in range(250):
        n = int(rng.integers(0, 11))
        boxes = _random_boxes(rng, n, canvas=30.0, lo=5.0, hi=25.0)
        scores = (rng.integers(0, 4, n) / 4).astype(np.float32)
        t = float(rng.choice([0.1, 0.3, 0.5, 0.7]))
        cls = rng.integers(0, 2, n).astype(np.int32) if trial % 3 == 0 else None
        offs = None
        if trial % 4 == 1:
            c = int(rng.integers(0, n + 1))
            offs = np.array([0, c, n], dtype=np.int64)
        want = oracle.brute_force(boxes, scores, t, cls, offs)
        np.testing.assert_array_equal(oracle.c_nms(boxes, scores, t, cls, offs), want)


def test_c_and_numpy_oracles_agree_on_many_seeded_inputs():
    for seed in range(400):
        n = [0, 1, 2, 5, 17, 63, 64, 65, 130, 300][seed % 10]
        w = workloads.random_small(seed, n, canvas=60.0,
                                   score_levels=[0, 4, 64][seed % 3],
                                   classes=[0, 3][seed % 2], images=[0, 3][(seed // 2) % 2])
        a = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
        b = oracle.np_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
        np.testing.assert_array_equal(a, b, err_msg=w.name)
        assert oracle.certify(w.boxes, w.scores, w.iou_threshold, a,
                              w.class_ids, w.batch_offsets) is None, w.name


@pytest.mark.parametrize("cfg", [1, 3])
def test_oracles_agree_on_small_configs(cfg):
    w = workloads.config(cfg, seed=0)
    a = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    b = oracle.np_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    np.testing.assert_array_equal(a, b)
    assert oracle.certify(w.boxes, w.scores, w.iou_threshold, a) is None


def test_error_statuses():
    boxes = np.float32([[0, 0, 1, 1], [0, 0, 2, 2]])
    scores = np.float32([0.5, 0.4])
    for fn in (oracle.c_nms, oracle.np_nms):
        with pytest.raises(oracle.OracleError) as e:
            fn(boxes, np.float32([np.nan, 0.1]), 0.5)
        assert e.value.status == "NONFINITE_INPUT"
        bad = boxes.copy()
        bad[1, 2] = np.inf
        with pytest.raises(oracle.OracleError) as e:
            fn(bad, scores, 0.5)
        assert e.value.status == "NONFINITE_INPUT"
        with pytest.raises(oracle.OracleError) as e:
            fn(boxes, scores, 0.5, None, np.array([0, 3], dtype=np.int64))
        assert e.value.status == "BAD_OFFSETS"
        with pytest.raises(oracle.OracleError) as e:
            fn(boxes, scores, 0.5, None, np.array([0, 2, 1, 2], dtype=np.int64))
        assert e.value.status == "BAD_OFFSETS"
        with pytest.raises(oracle.OracleError) as e:
            fn(boxes, scores, float("nan"))
        assert e.value.status == "INVALID_ARG"


def test_negative_zero_score_ties_positive_zero():
    boxes = np.float32([[0, 0, 10, 10], [0, 0, 10, 10], [50, 50, 60, 60]])
    scores = np.float32([-0.0, 0.0, -0.0])
    assert oracle.c_nms(boxes, scores, 0.5).tolist() == [0, 2]


def test_mask_rows_layout_pin():
    d = load_raw("layout_box5")
    boxes = np.float32(d["boxes"])
    scores = np.float32(d["scores"])
    order = oracle.stable_order(scores)
    np.testing.assert_array_equal(order, np.arange(len(scores)))
    m = oracle.mask_rows(boxes, d["iou_threshold"], order)
    assert m.shape == (130, 3)
    for row, word, val in d["expected_mask_words"]:
        assert int(m[row, word]) == int(val, 16), (row, word)


def _sweep_mask(m, n):
    removed = np.zeros(m.shape[1] * 64, dtype=bool)
    kept = []
    for p in range(n):
        if not removed[p]:
            kept.append(p)
            bits = np.unpackbits(m[p].view(np.uint8), bitorder="little").astype(bool)
            removed |= bits
    return np.asarray(kept, dtype=np.int64)


def test_mask_rows_sweep_reproduces_oracle():
    # the bitmask of the LeetCUDA page's Phase 1 followed by its Phase 2
    # sweep must give the oracle's result
    for seed in range(12):
        w = workloads.random_small(seed, [1, 63, 64, 65, 129, 200][seed % 6], canvas=50.0,
                                   score_levels=8)
        order = oracle.stable_order(w.scores)
        m = oracle.mask_rows(w.boxes, w.iou_threshold, order)
        # no bit at or below the diagonal
        for p in range(w.n):
            bits = np.unpackbits(m[p].view(np.uint8), bitorder="little")
            assert not bits[:p + 1].any()
        got = order[_sweep_mask(m, w.n)]
        np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))


def test_workloads_are_seeded_and_shaped():
    for cfg, n in ((1, 1024), (2, 8192), (3, 4096), (4, 64000)):
        a = workloads.config(cfg, 0)
        b = workloads.config(cfg, 0)
        c = workloads.config(cfg, 1)
        assert a.n == n and a.boxes.dtype == np.float32 and a.scores.dtype == np.float32
        assert a.sha256() == b.sha256() != c.sha256()
        assert np.all(a.boxes[:, 2] > a.boxes[:, 0]) and np.all(a.boxes[:, 3] > a.boxes[:, 1])
    w4 = workloads.config(4, 0)
    assert w4.class_ids.dtype == np.int32 and w4.class_ids.max() < 80
    assert w4.batch_offsets.tolist() == list(range(0, 64001, 4000))
    w3 = workloads.config(3, 0)
    assert np.unique(w3.scores).size <= 16


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin above
# ---------------------------------------------------------------------------

MUTANTS = [
    ("non-strict compare", "if (iou > iou_thresh) removed[j] = 1;",
     "if (iou >= iou_thresh) removed[j] = 1;"),
    ("ties by descending index", "if (score[idx[b]] > score[idx[a]])",
     "if (score[idx[b]] >= score[idx[a]])"),
    ("sorted positions returned", "keep_out[kept++] = i;", "keep_out[kept++] = p;"),
    ("+1 on box width", "float w = b[2] - b[0];", "float w = b[2] - b[0] + 1.0f;"),
    ("+1 on overlap height", "float h = fmax_plain(yy2 - yy1, 0.0f);",
     "float h = fmax_plain(yy2 - yy1 + 1.0f, 0.0f);"),
    ("overlap not clamped", "float w = fmax_plain(xx2 - xx1, 0.0f);", "float w = xx2 - xx1;"),
    ("union without the overlap", "float uni = (ai + aj) - inter;", "float uni = ai + aj;"),
    ("union summed in another order", "float uni = (ai + aj) - inter;",
     "float uni = ai + (aj - inter);"),
    ("min and max swapped", "float yy1 = fmax_plain(bi[1], bj[1]);",
     "float yy1 = fmin_plain(bi[1], bj[1]);"),
    ("wrong coordinate index", "float xx2 = fmin_plain(bi[2], bj[2]);",
     "float xx2 = fmin_plain(bi[3], bj[2]);"),
    ("float64 evaluation", "float uni = (ai + aj) - inter;\n    return inter / uni;",
     "double uni = ((double)ai + (double)aj) - (double)inter;\n    return (float)((double)inter / uni);"),
    ("fast NMS: removed boxes still suppress",
     "if (removed[i]) continue;\n        keep_out[kept++] = i;",
     "if (!removed[i]) keep_out[kept++] = i;"),
    ("class ignored", "if (class_ids != NULL && class_ids[j] != class_ids[i]) continue;", ""),
    ("image ignored", "if (image[j] != image[i]) continue;", ""),
    ("removal never recorded", "if (iou > iou_thresh) removed[j] = 1;", "(void)iou;"),
]


def _pins_pass(lib_path):
    """Run the pins against a given build of the C oracle; True if all pass."""
    try:
        for name, boxes, scores, t, cls, offs, expected in CASES:
            got = oracle.c_nms(boxes, scores, t, cls, offs, lib_path=lib_path)
            if not np.array_equal(got, expected):
                return False
        d = load_raw("fp32_union_rounding")
        iou = oracle.c_pair_iou(np.float32(d["boxes"]), np.array([0]), np.array([1]),
                                lib_path=lib_path)[0]
        if iou != np.float32(d["expected_iou_f32"]):
            return False
        boxes = np.float32([p for a, b, _ in IOU_PAIRS for p in (a, b)])
        a = np.arange(0, 2 * len(IOU_PAIRS), 2)
        if not np.array_equal(oracle.c_pair_iou(boxes, a, a + 1, lib_path=lib_path),
                              np.float32([v for _, _, v in IOU_PAIRS])):
            return False
    except oracle.OracleError:
        return False
    return True


def test_unmutated_build_passes_pins(tmp_path):
    src = os.path.join(os.path.dirname(oracle.__file__), "nms_oracle.c")
    out = str(tmp_path / "liboracle_copy.so")
    oracle.build_c_oracle(force=True, src=src, out=out)
    assert _pins_pass(out)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes(mutant, tmp_path):
    label, old, new = mutant
    src = os.path.join(os.path.dirname(oracle.__file__), "nms_oracle.c")
    with open(src) as f:
        text = f.read()
    assert text.count(old) == 1, label
    msrc = tmp_path / "mutant.c"
    msrc.write_text(text.replace(old, new))
    out = str(tmp_path / "libmutant.so")
    oracle.build_c_oracle(force=True, src=str(msrc), out=out)
    assert not _pins_pass(out), "pins did not catch: " + label
