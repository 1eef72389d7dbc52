"""Pins for the oracle's certificate checker ``oracle.certify`` (no GPU).

A kept list K is the greedy result iff (I1) K is strictly increasing in
sorted position, (I2) no kept box is overlapped above the threshold by an
earlier kept box of its group, and (I3) every box left out is overlapped
above the threshold by an earlier kept box of its group ("LeetCUDA 14-nms",
introduction and algorithm steps; the group rule is the class check of
"YOLOv5 post-processing GPU port", section 2.2).  Each case below builds a
wrong list from a hand-worked fixture and must be rejected with the right
property; the right list must be accepted.  ``test_planted_certify_mistakes``
runs the same cases against copies of ``certify`` with one plausible slip
each and shows that every slip fails at least one case.
"""
import inspect
import textwrap

import numpy as np
import pytest

import oracle
import oracle.reference as ref

F = np.float32

# Chain (hand-worked): IoU(0,1) = IoU(1,2) = 50/150 = 1/3 > 0.3, IoU(0,2) = 0.
# Greedy keeps [0, 2]; Fast NMS would keep [0].
CHAIN = (F([[0, 0, 10, 10], [5, 0, 15, 10], [10, 0, 20, 10]]), F([0.9, 0.8, 0.7]), 0.3)
# Nested half box: inter 50, union 100, IoU exactly 0.5.
HALF = (F([[0, 0, 10, 10], [0, 0, 10, 5]]), F([0.9, 0.8]))
# Scores ascending in index: sorted positions are the reverse of the indices.
# Boxes 2 and 1 coincide (IoU 1), box 0 is far away.
REV = (F([[100, 100, 110, 110], [0, 0, 10, 10], [0, 0, 10, 10]]), F([0.1, 0.2, 0.3]), 0.5)
# Two identical boxes: one group removes the second, different classes or
# images keep both.
TWIN = F([[0, 0, 10, 10], [0, 0, 10, 10]])
TWIN_S = F([0.9, 0.8])

# (name, call arguments, kept list, expected verdict prefix or None)
CASES = [
    ("chain_right", (*CHAIN, [0, 2]), {}, None),
    ("chain_drop_kept", (*CHAIN, [0]), {}, "I3"),          # Fast NMS's answer
    ("chain_add_removed", (*CHAIN, [0, 1, 2]), {}, "I2"),
    ("chain_swapped", (*CHAIN, [2, 0]), {}, "I1"),
    ("chain_repeated", (*CHAIN, [0, 0, 2]), {}, "I1: repeated"),
    ("chain_out_of_range", (*CHAIN, [0, 3]), {}, "I1"),
    ("chain_negative_index", (*CHAIN, [-1, 0, 2]), {}, "I1"),
    ("chain_empty", (*CHAIN, []), {}, "I3"),
    # at t = 0.5 the exact-0.5 pair does not suppress (strict >)
    ("half_at_t_right", (*HALF, 0.5, [0, 1]), {}, None),
    ("half_at_t_drop", (*HALF, 0.5, [0]), {}, "I3"),
    ("half_below_t_right", (*HALF, 0.49, [0]), {}, None),
    ("half_below_t_add", (*HALF, 0.49, [0, 1]), {}, "I2"),
    # sorted positions, not input indices, decide I1
    ("rev_right", (*REV, [2, 0]), {}, None),
    ("rev_index_order", (*REV, [0, 2]), {}, "I1"),
    ("rev_keeps_removed", (*REV, [2, 1, 0]), {}, "I2"),
    # groups
    ("class_right", (TWIN, TWIN_S, 0.5, [0, 1]), {"class_ids": np.int32([3, 4])}, None),
    ("class_drop", (TWIN, TWIN_S, 0.5, [0]), {"class_ids": np.int32([3, 4])}, "I3"),
    ("same_class_right", (TWIN, TWIN_S, 0.5, [0]), {"class_ids": np.int32([7, 7])}, None),
    ("same_class_add", (TWIN, TWIN_S, 0.5, [0, 1]), {"class_ids": np.int32([7, 7])}, "I2"),
    ("image_right", (TWIN, TWIN_S, 0.5, [0, 1]), {"batch_offsets": np.int64([0, 1, 2])}, None),
    ("image_drop", (TWIN, TWIN_S, 0.5, [1]), {"batch_offsets": np.int64([0, 1, 2])}, "I3"),
]


def _run(certify_fn, case):
    name, args, kw, want = case
    boxes, scores, t, keep = args
    return certify_fn(boxes, scores, t, np.asarray(keep, dtype=np.int64), **kw)


def _verdict_ok(got, want):
    if want is None:
        return got is None
    return got is not None and got.startswith(want)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_certify_verdicts(case):
    got = _run(oracle.certify, case)
    assert _verdict_ok(got, case[3]), "%s: got %r, want %r" % (case[0], got, case[3])


def test_certify_accepts_oracle_results_and_rejects_single_edits():
    """On seeded random inputs: the oracle's list is accepted; removing any
    one kept box, or adding any one removed box, is rejected."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        n = int(rng.integers(5, 40))
        xy = rng.uniform(0, 60, (n, 2))
        wh = rng.uniform(5, 30, (n, 2))
        boxes = F(np.concatenate([xy, xy + wh], axis=1))
        scores = F(rng.integers(1, 6, n) / 5.0)   # ties
        keep = oracle.c_nms(boxes, scores, 0.4)
        assert oracle.certify(boxes, scores, 0.4, keep) is None
        for k in range(keep.size):
            assert oracle.certify(boxes, scores, 0.4, np.delete(keep, k)) is not None
        removed = np.setdiff1d(np.arange(n), keep)
        order = oracle.stable_order(scores)
        pos = np.empty(n, np.int64)
        pos[order] = np.arange(n)
        for j in removed[:5]:
            bad = np.array(sorted(list(keep) + [j], key=lambda i: pos[i]), dtype=np.int64)
            assert oracle.certify(boxes, scores, 0.4, bad) is not None


# Plausible slips in the checker: each replaces one fragment of its source.
MUTANTS = {
    "non_strict": ("> t]", ">= t]"),
    "no_i2": ("if np.any(covered & in_k):", "if False:"),
    "no_i3": ("if np.any(~covered & ~in_k):", "if False:"),
    "no_order_check": ("if np.any(np.diff(kp) <= 0):", "if False:"),
    "no_range_check": ("if keep.size and (keep.min() < 0 or keep.max() >= n):",
                       "if False:"),
    "no_repeat_check": ("if np.unique(keep).size != keep.size:", "if False:"),
    "groups_ignored": ("(img[later] == img[i]) & (cls[later] == cls[i])",
                       "np.ones(later.size, dtype=bool)"),
    "input_order": ("kp = pos[keep]", "kp = keep"),
    "always_none": ('    """Return None', '    return None\n    """Return None'),
}


def _mutant(fragment, replacement):
    src = textwrap.dedent(inspect.getsource(ref.certify))
    assert fragment in src, fragment
    ns = dict(vars(ref))
    exec(compile(src.replace(fragment, replacement, 1), "<certify mutant>", "exec"), ns)
    return ns["certify"]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_certify_mistakes(mutant):
    fn = _mutant(*MUTANTS[mutant])
    failures = []
    for case in CASES:
        try:
            got = _run(fn, case)
        except Exception as e:  # a slip that crashes is caught as well
            failures.append((case[0], repr(e)))
            continue
        if not _verdict_ok(got, case[3]):
            failures.append((case[0], got))
    assert failures, "the planted mistake %s passed every certify pin" % mutant
