"""Pins of the Matrix NMS oracle (CPU only).

The C oracle (``oracle.c_matrix_nms``) and the naive matrix formulation in
numpy (``oracle.np_matrix_nms``) are checked against hand-computed fixtures
(tests/golden/matrix/, each with its citation and arithmetic), closed forms
and each other; planted mistakes in the C oracle must each fail a pin."""
import glob
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "matrix")


def _cases():
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        d = json.load(open(path))
        assert d["citation"]
        name = os.path.splitext(os.path.basename(path))[0]
        for k, c in enumerate(d["cases"]):
            out.append(("%s[%d]" % (name, k), np.float32(d["boxes"]), np.float32(d["scores"]),
                        float(c["score_threshold"]), float(c.get("sigma", d.get("sigma", 0.5))),
                        np.asarray(c["expected_keep"], dtype=np.int64)))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_golden_c_oracle(case):
    _, boxes, scores, t, sigma, want = case
    np.testing.assert_array_equal(oracle.c_matrix_nms(boxes, scores, t, sigma), want)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_golden_naive_matrix_formulation(case):
    _, boxes, scores, t, sigma, want = case
    np.testing.assert_array_equal(oracle.np_matrix_nms(boxes, scores, t, sigma), want)


def _grid(k, step=20.0, size=10.0):
    xy = np.array([(step * (i % 8), step * (i // 8)) for i in range(k)], dtype=np.float64)
    return np.float32(np.concatenate([xy, xy + size], axis=1))


def test_closed_form_disjoint_boxes_keep_by_score_alone():
    # no overlaps: every O and O_max is 0, every decay is exp(0) = 1, so a box
    # stays iff its score reaches t; a score equal to t stays (the drop test
    # is strict), including for boxes with fathers
    boxes = _grid(12)
    scores = np.float32([0.9, 0.2, 0.5, 0.5, 0.05, 0.7, 0.3, 0.3, 0.6, 0.1, 0.3, 0.8])
    t = 0.3
    want = np.argsort(-scores, kind="stable")
    want = want[scores[want] >= np.float32(t)]
    for sigma in (0.5, 2.0):
        np.testing.assert_array_equal(oracle.c_matrix_nms(boxes, scores, t, sigma), want)
        np.testing.assert_array_equal(oracle.np_matrix_nms(boxes, scores, t, sigma), want)


def test_closed_form_top_box_below_threshold_drops_everything():
    boxes = _grid(5)
    scores = np.float32([0.2, 0.1, 0.25, 0.05, 0.15])
    assert oracle.c_matrix_nms(boxes, scores, 0.3).size == 0
    assert oracle.np_matrix_nms(boxes, scores, 0.3).size == 0


def test_closed_form_wide_sigma_keeps_by_score():
    # sigma -> infinity sends every exponent to 0
    w = workloads.random_small(41, 200, canvas=80.0)
    want = np.argsort(-w.scores, kind="stable")
    want = want[w.scores[want] >= np.float32(0.4)]
    np.testing.assert_array_equal(oracle.c_matrix_nms(w.boxes, w.scores, 0.4, 1e30), want)


def test_threshold_monotone():
    w = workloads.random_small(43, 300, canvas=120.0)
    prev = None
    for t in (0.05, 0.1, 0.2, 0.3, 0.5, 0.8):
        k = set(oracle.c_matrix_nms(w.boxes, w.scores, t).tolist())
        if prev is not None:
            assert k <= prev
        prev = k


def test_c_and_naive_formulations_agree_on_seeded_inputs():
    for seed in range(60):
        n = [1, 2, 3, 17, 64, 65, 130, 257][seed % 8]
        w = workloads.random_small(3000 + seed, n, canvas=3.0 * np.sqrt(n) + 25,
                                   score_levels=[0, 8][seed % 2])
        t = [0.05, 0.2, 0.4][seed % 3]
        sigma = [0.5, 0.5, 2.0, 0.1][seed % 4]
        got, border = oracle.c_matrix_nms(w.boxes, w.scores, t, sigma, return_borderline=True)
        assert border == 0
        np.testing.assert_array_equal(got, oracle.np_matrix_nms(w.boxes, w.scores, t, sigma))


def test_error_statuses():
    b = np.float32([[0, 0, 1, 1], [2, 2, 3, 3]])
    s = np.float32([0.5, 0.4])
    for bad, status in [((b, np.float32([np.nan, 0.1]), 0.1, 0.5), "NONFINITE_INPUT"),
                        ((np.float32([[0, 0, np.inf, 1], [2, 2, 3, 3]]), s, 0.1, 0.5),
                         "NONFINITE_INPUT"),
                        ((np.float32([[2, 0, 1, 1], [2, 2, 3, 3]]), s, 0.1, 0.5), "BAD_BOXES"),
                        ((b, s, 0.1, 0.0), "INVALID_ARG"),
                        ((b, s, float("nan"), 0.5), "INVALID_ARG")]:
        with pytest.raises(oracle.OracleError) as e:
            oracle.c_matrix_nms(*bad)
        assert e.value.status == status
    assert oracle.c_matrix_nms(np.zeros((0, 4), np.float32), np.zeros(0, np.float32), 0.1).size == 0


# ---------------------------------------------------------------------------
# planted mistakes in the C oracle's Matrix NMS: each must fail a pin above
# ---------------------------------------------------------------------------

MUTANTS = [
    ("no compensation by the father's own overlap",
     "double x = ((double)omax[p] * (double)omax[p] - (double)o * (double)o) / sigma;",
     "double x = (0.0 - (double)o * (double)o) / sigma;"),
    ("sigma multiplies",
     "double x = ((double)omax[p] * (double)omax[p] - (double)o * (double)o) / sigma;",
     "double x = ((double)omax[p] * (double)omax[p] - (double)o * (double)o) * sigma;"),
    ("squares dropped",
     "double x = ((double)omax[p] * (double)omax[p] - (double)o * (double)o) / sigma;",
     "double x = ((double)omax[p] - (double)o) / sigma;"),
    ("non-strict drop", "if (cand < t) drop = 1;", "if (cand <= t) drop = 1;"),
    ("score rule missing", "int drop = s < t;", "int drop = 0;"),
    ("omax over children too", "for (int64_t p = 0; p < q; ++p) {\n            const int64_t i = order[p];\n            float o = overlap_or_zero",
     "for (int64_t p = 0; p < n; ++p) {\n            if (p == q) continue;\n            const int64_t i = order[p];\n            float o = overlap_or_zero"),
    ("decay factor inverted", "double cand = exp(x) * s;", "double cand = exp(-x) * s;"),
    ("sorted positions returned", "if (!drop) keep_out[kept++] = j;",
     "if (!drop) keep_out[kept++] = q;"),
]


def _pins_pass(lib_path):
    try:
        for _, boxes, scores, t, sigma, want in CASES:
            if not np.array_equal(oracle.c_matrix_nms(boxes, scores, t, sigma, lib_path=lib_path),
                                  want):
                return False
        boxes = _grid(12)
        scores = np.float32([0.9, 0.2, 0.5, 0.5, 0.05, 0.7, 0.3, 0.3, 0.6, 0.1, 0.3, 0.8])
        want = np.argsort(-scores, kind="stable")
        want = want[scores[want] >= np.float32(0.3)]
        if not np.array_equal(oracle.c_matrix_nms(boxes, scores, 0.3, lib_path=lib_path), want):
            return False
        b5 = _grid(5)
        if oracle.c_matrix_nms(b5, np.float32([0.2, 0.1, 0.25, 0.05, 0.15]), 0.3,
                               lib_path=lib_path).size:
            return False
    except oracle.OracleError:
        return False
    return True


def test_unmutated_build_passes_matrix_pins(tmp_path):
    src = os.path.join(os.path.dirname(oracle.__file__), "nms_oracle.c")
    out = str(tmp_path / "liboracle_copy.so")
    oracle.build_c_oracle(force=True, src=src, out=out)
    assert _pins_pass(out)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_matrix_mistakes(mutant, tmp_path):
    label, old, new = mutant
    src = os.path.join(os.path.dirname(oracle.__file__), "nms_oracle.c")
    text = open(src).read()
    assert text.count(old) == 1, label
    msrc = tmp_path / "mutant.c"
    msrc.write_text(text.replace(old, new))
    out = str(tmp_path / "libmutant.so")
    oracle.build_c_oracle(force=True, src=str(msrc), out=out)
    assert not _pins_pass(out), "pins did not catch: " + label
