"""The one-launch path for small inputs (one image of 1 to 4096 boxes: sort,
mask, sweep and output in a single launch; nms_f32_ex with
NMS_FLAG_ONE_LAUNCH), against the oracle and against the multi-launch path,
including the case where it gives up (a row tile with more nonzero mask
words than its list holds) and the call runs the multi-launch path instead.

Why it exists: the LeetCUDA 14-nms page, measured results, loses at 1024 and
2048 boxes to fixed per-launch costs.  Which path ran is visible in the
stage times: the one-launch path records its whole time as the mask stage
(the sort stage reads 0); the multi-launch path times its sort."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu


def _g():
    import greedy_iou_nms_amd as g
    return g


def _run(w, workspace=None, one_launch=True, fuse=True):
    g = _g()
    dev = device()
    b = to_dev(np.asarray(w.boxes, np.float32).reshape(-1, 4), dev)
    s = to_dev(np.asarray(w.scores, np.float32), dev)
    keep, st = g.nms_profiled(b, s, w.iou_threshold, workspace=workspace, fuse=fuse,
                              one_launch=one_launch)
    return keep.cpu().numpy(), st


def test_plan_names_the_one_launch_path():
    g = _g()
    for n in (1, 64, 1000, 4096):
        assert g.debug_plan(n)["small"] == 1, n
    assert g.debug_plan(4097)["small"] == 0
    assert g.debug_plan(1000, 2)["small"] == 0          # two images
    assert g.debug_plan(1000, 1, True)["small"] == 0    # class ids


@pytest.mark.parametrize("cfg,seed", [(1, 0), (1, 1), (1, 2), (3, 0), (3, 1), (3, 2)])
def test_configs_one_launch_vs_multi_launch_vs_oracle(cfg, seed):
    w = workloads.config(cfg, seed)
    note("small path cfg=%d seed=%d" % (cfg, seed))
    one, st1 = _run(w)
    multi, st2 = _run(w, one_launch=False)
    plain = _g().nms(to_dev(w.boxes, device()), to_dev(w.scores, device()), w.iou_threshold,
                     one_launch=True).cpu().numpy()
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold)
    np.testing.assert_array_equal(one, want)
    np.testing.assert_array_equal(multi, want)
    np.testing.assert_array_equal(plain, want)
    assert st1["sort"] == 0.0 and st1["mask"] > 0.0, st1   # the one launch ran
    assert st2["sort"] > 0.0, st2


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 129, 1000, 2047, 2049, 4095, 4096])
def test_ragged_sizes(n):
    w = workloads.random_small(7000 + n, n, canvas=40.0 + n / 6.0)
    note("small path ragged n=%d t=%r" % (n, w.iou_threshold))
    got, st = _run(w)
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))
    assert st["sort"] == 0.0, st


@pytest.mark.parametrize("n,levels", [(1024, 4), (4096, 16), (3000, 1)])
def test_tied_scores(n, levels):
    # equal scores keep input order; one level: every score equal
    w = workloads.random_small(8100 + n, n, canvas=60.0 + n / 8.0, score_levels=levels)
    if levels == 1:
        w.scores = np.full(n, 0.25, np.float32)
    note("small path ties n=%d levels=%d" % (n, levels))
    got, _ = _run(w)
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))


def test_overflowing_tile_list_falls_back_to_the_multi_launch_path():
    # 4096 nearly equal boxes: every pair overlaps, the first row tile has
    # 64 x 64 nonzero words (more than its list holds), the one launch gives
    # up and the call runs the stages separately
    n = 4096
    rng = np.random.default_rng(5)
    base = np.array([100.0, 100.0, 200.0, 180.0])
    boxes = (base[None, :] + rng.uniform(-1.0, 1.0, (n, 4))).astype(np.float32)
    w = workloads.Workload("dense_%d" % n, boxes, rng.random(n).astype(np.float32), 0.5)
    note("small path overflow fallback n=%d" % n)
    got, st = _run(w)
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold)
    np.testing.assert_array_equal(got, want)
    assert want.size < 4
    assert st["sort"] > 0.0, st    # the multi-launch path produced the result


def test_dense_but_within_the_lists():
    # 2048 boxes in heavy overlap: at most 32 words per row, 2048 per tile,
    # so the lists never overflow and the one launch stands
    n = 2048
    rng = np.random.default_rng(6)
    base = np.array([10.0, 10.0, 90.0, 70.0])
    boxes = (base[None, :] + rng.uniform(-3.0, 3.0, (n, 4))).astype(np.float32)
    w = workloads.Workload("dense_%d" % n, boxes, rng.random(n).astype(np.float32), 0.6)
    note("small path dense within lists n=%d" % n)
    got, st = _run(w)
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))
    assert st["sort"] == 0.0, st


@pytest.mark.parametrize("t", [0.0, 1.0, -0.5, 1.5, float(np.float32(1e-30))])
def test_thresholds_outside_the_fast_test(t):
    w = workloads.random_small(8200, 3000, canvas=300.0)
    w.iou_threshold = t
    note("small path threshold %r" % t)
    got, _ = _run(w)
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, t))


def test_degenerate_and_inverted_boxes():
    # boxes with x1 >= x2 or y1 >= y2 (zero or negative extent) take the
    # mask's literal form
    w = workloads.random_small(8300, 2500, canvas=200.0)
    b = w.boxes.copy()
    b[::7, 2] = b[::7, 0]                  # zero width
    b[3::11, [0, 2]] = b[3::11, [2, 0]]    # inverted in x
    b[5::13, [1, 3]] = b[5::13, [3, 1]]    # inverted in y
    w.boxes = b
    note("small path degenerate boxes n=%d" % w.n)
    got, st = _run(w)
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))
    assert st["sort"] == 0.0, st


def test_errors_then_a_good_call_on_the_same_workspace():
    g = _g()
    dev = device()
    w = workloads.config(1, 3)
    ws = g.Workspace(dev)
    bad = w.scores.copy()
    bad[77] = np.nan
    note("small path nan score then good call")
    with pytest.raises(g.NMSError, match="NONFINITE"):
        g.nms(to_dev(w.boxes, dev), to_dev(bad, dev), 0.5, workspace=ws, one_launch=True)
    boxes = w.boxes.copy()
    boxes[5, 2] = np.inf
    with pytest.raises(g.NMSError, match="NONFINITE"):
        g.nms(to_dev(boxes, dev), to_dev(w.scores, dev), 0.5, workspace=ws, one_launch=True)
    got, _ = _run(w, workspace=ws)
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))


def test_repeated_calls_alternating_inputs_and_workspaces():
    # every call has its own epoch: what one call leaves in a workspace
    # (slots, counters, lists) must never pass for the next call's
    g = _g()
    dev = device()
    ws = [g.Workspace(dev), g.Workspace(dev)]
    cases = [workloads.config(1, 4), workloads.config(3, 4),
             workloads.random_small(8400, 333, canvas=90.0)]
    wants = [oracle.c_nms(w.boxes, w.scores, w.iou_threshold) for w in cases]
    dev_in = [(to_dev(w.boxes, dev), to_dev(w.scores, dev), w.iou_threshold) for w in cases]
    note("small path 60 alternating calls")
    for i in range(60):
        k = (i * 7) % 3
        b, s, t = dev_in[k]
        got = g.nms(b, s, t, workspace=ws[i % 2], one_launch=True).cpu().numpy()
        np.testing.assert_array_equal(got, wants[k], err_msg="call %d case %d" % (i, k))
