"""nms_f32_static, the entry point that allocates nothing (its scratch is a
static device array in the library): through the C ABI it must return what
nms_f32 returns, call after call, also when a call follows a larger one on
the same scratch, and refuse sizes beyond its scratch."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu


def _g():
    import greedy_iou_nms_amd as g
    return g


def _both(w, dev):
    g = _g()
    b = to_dev(w.boxes, dev)
    s = to_dev(w.scores, dev)
    c = to_dev(w.class_ids, dev)
    o = to_dev(w.batch_offsets, dev)
    got = g.nms_static(b, s, w.iou_threshold, c, o).cpu().numpy()
    want = g.nms(b, s, w.iou_threshold, c, o).cpu().numpy()
    return got, want


def test_static_entry_point_matches_nms_f32_on_consecutive_calls():
    dev = device()
    big = workloads.config(2, 0)                       # 8192 clustered boxes
    small = workloads.random_small(77, 1500, canvas=200.0, score_levels=6)
    grouped = workloads.random_small(78, 3000, canvas=150.0, score_levels=8, classes=3,
                                     images=2)
    for w in (big, small, grouped, workloads.config(3, 1), workloads.config(1, 2)):
        note("static entry point %s n=%d" % (w.name, w.n))
        got, want = _both(w, dev)
        np.testing.assert_array_equal(got, want)
        np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold,
                                                        w.class_ids, w.batch_offsets))


def test_static_entry_point_largest_and_too_large():
    g = _g()
    dev = device()
    n = g.STATIC_MAX_BOXES
    w = workloads.random_small(79, n, canvas=60.0 + n / 8.0)
    note("static entry point n=%d" % n)
    got, want = _both(w, dev)
    np.testing.assert_array_equal(got, want)
    w2 = workloads.random_small(80, n + 1, canvas=60.0 + n / 8.0)
    with pytest.raises(g.NMSError) as e:
        g.nms_static(to_dev(w2.boxes, dev), to_dev(w2.scores, dev), 0.5)
    assert e.value.status == "NMS_TOO_LARGE"
    # the next call still works
    w3 = workloads.config(1, 0)
    got, want = _both(w3, dev)
    np.testing.assert_array_equal(got, want)


def test_static_entry_point_reports_device_errors():
    g = _g()
    dev = device()
    w = workloads.config(1, 0)
    s = w.scores.copy()
    s[3] = np.nan
    with pytest.raises(g.NMSError) as e:
        g.nms_static(to_dev(w.boxes, dev), to_dev(s, dev), 0.5)
    assert e.value.status == "NMS_NONFINITE_INPUT"
    got, want = _both(w, dev)
    np.testing.assert_array_equal(got, want)
