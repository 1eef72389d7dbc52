"""The radix sort in one launch (team_sort.hip: a team of resident
workgroups runs every pass) against the stable orders it must produce, and
end to end against the oracle and against the sort with one launch per pass
(NMS_FLAG_PASS_SORT).

The order is the page's step 1 ("LeetCUDA 14-nms", algorithm and data flow:
a stable descending sort, equal scores in input order); grouped input sorts
by (image, class) first ("YOLOv5 post-processing", section 2.2), and keeps
the plain score order for the output."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _g():
    import greedy_iou_nms_amd as g
    return g


def _tied_scores(n, seed):
    # few distinct values (long runs of ties), signed zeros, a few singletons
    rng = np.random.default_rng(seed)
    s = (rng.integers(-8, 8, n) / 4).astype(np.float32)
    s[rng.integers(0, n, max(1, n // 10))] = -0.0
    s[rng.integers(0, n, max(1, n // 10))] = rng.random(max(1, n // 10)).astype(np.float32)
    return s


def test_plan_names_the_team_sort():
    g = _g()
    for n in (16385, 65536, 131072):
        assert g.debug_plan(n)["team_sort"] == 1, n
    for n in (1, 16384, 131073, 512000):
        assert g.debug_plan(n)["team_sort"] == 0, n
    for n in (1, 1000, 16384, 64000, 131072):
        assert g.debug_plan(n, 16, True)["team_sort"] == 1, n
    assert g.debug_plan(131073, 2, True)["team_sort"] == 0


# tile sizes of 1024, 2048 and 4096 boxes per member, full and ragged; above
# 131072 the sort with one launch per pass
@pytest.mark.parametrize("n", [16385, 20000, 32768, 32769, 65535, 65536, 65537, 100003, 131072,
                               131073, 262144])
def test_one_image_order(n):
    dev = device()
    scores = _tied_scores(n, n)
    note("team sort one image n=%d" % n)
    order, _ = _g().debug_order(to_dev(scores, dev))
    np.testing.assert_array_equal(order.cpu().numpy(), np.argsort(-scores, kind="stable"))


def test_one_image_distinct_and_uniform_scores():
    dev = device()
    rng = np.random.default_rng(3)
    for n in (40000, 65536):
        scores = rng.random(n).astype(np.float32)
        note("team sort uniform n=%d" % n)
        order, _ = _g().debug_order(to_dev(scores, dev))
        np.testing.assert_array_equal(order.cpu().numpy(), np.argsort(-scores, kind="stable"))


@pytest.mark.parametrize("value", [0.5, -0.0, 0.0])
def test_every_score_equal(value):
    # every digit of every key is the same: all passes would be skipped, the
    # last one runs anyway and writes the input order
    dev = device()
    n = 70001
    scores = np.full(n, value, np.float32)
    note("team sort equal scores %r" % value)
    order, _ = _g().debug_order(to_dev(scores, dev))
    np.testing.assert_array_equal(order.cpu().numpy(), np.arange(n))


def _grouped_want(scores, cls, offs):
    n = scores.shape[0]
    img, c = oracle.groups_of(n, cls, offs)
    return (np.lexsort((np.arange(n), -scores, c, img)),
            np.argsort(-scores, kind="stable"))


@pytest.mark.parametrize("n,images,classes", [
    (1, 1, 3), (7, 2, 0), (1000, 1, 80), (5000, 3, 5), (16384, 16, 80), (64000, 16, 80),
    (70000, 300, 0), (100003, 2, 1000), (200000, 64, 7)])
def test_grouped_order(n, images, classes):
    dev = device()
    rng = np.random.default_rng(n + images)
    scores = _tied_scores(n, n + 1)
    cls = None
    if classes:
        # signed class ids, some negative
        cls = rng.integers(-3, classes, n).astype(np.int32)
    offs = None
    if images > 1 or cls is None:
        cuts = np.sort(rng.integers(0, n + 1, max(images, 1) - 1))
        offs = np.concatenate([[0], cuts, [n]]).astype(np.int64)
    note("team sort grouped n=%d images=%d classes=%d" % (n, images, classes))
    order, sorder = _g().debug_order(to_dev(scores, dev), to_dev(cls, dev), to_dev(offs, dev))
    want, swant = _grouped_want(scores, cls, offs)
    np.testing.assert_array_equal(order.cpu().numpy(), want)
    np.testing.assert_array_equal(sorder.cpu().numpy(), swant)


@pytest.mark.parametrize("sizes", [[4096, 100, 4096, 1], [4096, 4097], [0, 3000, 0, 2500],
                                   [4096] * 20])
def test_grouped_images_at_the_lds_limit(sizes):
    # images of at most 4096 boxes are each sorted in LDS by one block; one
    # larger image sends the whole input through the team's passes
    dev = device()
    n = int(sum(sizes))
    rng = np.random.default_rng(len(sizes) + n)
    scores = _tied_scores(n, n + 2)
    cls = rng.integers(0, 90, n).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    note("team sort grouped, image sizes %s" % sizes[:4])
    order, sorder = _g().debug_order(to_dev(scores, dev), to_dev(cls, dev), to_dev(offs, dev))
    want, swant = _grouped_want(scores, cls, offs)
    np.testing.assert_array_equal(order.cpu().numpy(), want)
    np.testing.assert_array_equal(sorder.cpu().numpy(), swant)


def test_grouped_every_key_equal():
    dev = device()
    n = 30000
    scores = np.full(n, 0.25, np.float32)
    cls = np.full(n, 4, np.int32)
    note("team sort grouped, every key equal")
    order, sorder = _g().debug_order(to_dev(scores, dev), to_dev(cls, dev))
    np.testing.assert_array_equal(order.cpu().numpy(), np.arange(n))
    np.testing.assert_array_equal(sorder.cpu().numpy(), np.arange(n))


def _nms(w, pass_sort, workspace=None):
    dev = device()
    return _g().nms(to_dev(w.boxes, dev), to_dev(w.scores, dev), w.iou_threshold,
                    to_dev(w.class_ids, dev), to_dev(w.batch_offsets, dev),
                    workspace=workspace, pass_sort=pass_sort).cpu().numpy()


@pytest.mark.parametrize("cfg,seed", [(2, 0), (3, 1), (4, 0), (4, 1), (5, 0), (5, 1)])
def test_end_to_end_team_vs_pass_sort_vs_oracle(cfg, seed):
    w = workloads.config(cfg, seed)
    note("team vs pass sort cfg=%d seed=%d" % (cfg, seed))
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    np.testing.assert_array_equal(_nms(w, False), want)
    np.testing.assert_array_equal(_nms(w, True), want)


@pytest.mark.parametrize("images", [1, 2, 5, 32, 33])
def test_merged_images_end_to_end(images):
    # Images of at most 4096 boxes, each sorted on its own beside the team's
    # score passes, some empty; scores in few levels, so equal scores across
    # images are common: the earlier image's box (the smaller index) must
    # come first in the output.
    rng = np.random.default_rng(500 + images)
    sizes = rng.integers(0, 900, images)
    sizes[rng.integers(0, images)] = 0          # an empty image
    n = int(sizes.sum())
    base = workloads.random_small(600 + images, max(n, 1), canvas=300.0, score_levels=6,
                                  classes=5)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    w = workloads.Workload("merge_%d" % images, base.boxes[:n], base.scores[:n], 0.5,
                           base.class_ids[:n], offs)
    note("merged images=%d n=%d" % (images, n))
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    np.testing.assert_array_equal(_nms(w, False), want)


def test_one_image_with_classes_end_to_end():
    # no batch offsets: one image of classes, sorted on its own if small
    for n in (3000, 4096, 4097):
        w = workloads.random_small(700 + n, n, canvas=200.0, score_levels=8, classes=12)
        note("one image with classes n=%d" % n)
        want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, None)
        np.testing.assert_array_equal(_nms(w, False), want)


def test_one_large_group_end_to_end():
    # one image, one class, 40000 boxes: a grouped call whose band is wider
    # than the grouped sweep's window
    w = workloads.config(5, 2)
    n = 40000
    w = workloads.Workload("one_group_40000", w.boxes[:n].copy(), w.scores[:n].copy(),
                           w.iou_threshold, np.full(n, 9, np.int32), np.array([0, n], np.int64))
    note("team sort one large group")
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    np.testing.assert_array_equal(_nms(w, False), want)


def test_nonfinite_scores_and_boxes_are_reported():
    g = _g()
    w = workloads.config(4, 2)
    s = w.scores.copy()
    s[1234] = np.nan
    note("team sort NaN score (grouped)")
    with pytest.raises(g.NMSError, match="NONFINITE"):
        _nms(workloads.Workload("nan", w.boxes, s, w.iou_threshold, w.class_ids,
                                w.batch_offsets), False)
    w5 = workloads.config(5, 0)
    b = w5.boxes.copy()
    b[60001, 2] = np.inf
    note("team sort infinite box (one image)")
    with pytest.raises(g.NMSError, match="NONFINITE"):
        _nms(workloads.Workload("inf", b, w5.scores, w5.iou_threshold), False)
    offs = w.batch_offsets.copy()
    offs[3], offs[4] = offs[4], offs[3] - 1
    note("team sort bad offsets")
    with pytest.raises(g.NMSError, match="OFFSETS"):
        _nms(workloads.Workload("offs", w.boxes, w.scores, w.iou_threshold, w.class_ids,
                                offs), False)
    # and the next call on the same device is unaffected
    np.testing.assert_array_equal(
        _nms(w, False),
        oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets))


def test_repeated_calls_alternating_inputs_on_one_workspace():
    # every call tags its words anew: what one call left must never pass
    # for the next call's
    g = _g()
    dev = device()
    ws = g.Workspace(dev)
    cases = [workloads.config(4, 3), workloads.config(5, 3),
             workloads.Workload("ties", workloads.config(5, 4).boxes[:20000],
                                _tied_scores(20000, 5), 0.5)]
    wants = [oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
             for w in cases]
    note("team sort 30 alternating calls")
    for i in range(30):
        k = (i * 7) % 3
        np.testing.assert_array_equal(_nms(cases[k], False, ws), wants[k],
                                      err_msg="call %d case %d" % (i, k))


@pytest.mark.parametrize("fill", [0xFF, 0x00])
def test_workspace_contents_do_not_matter(fill):
    g = _g()
    dev = device()
    w = workloads.config(5, 5)
    ws = g.Workspace(dev)
    buf = ws.get(g.workspace_size(w.n, 0, False), dev)
    buf.fill_(fill)
    note("team sort workspace filled with %#x" % fill)
    np.testing.assert_array_equal(_nms(w, False, ws),
                                  oracle.c_nms(w.boxes, w.scores, w.iou_threshold))


# ---------------------------------------------------------------- sample sort
# One image of 16,385 to 131,072 boxes is sorted by sample sort (samples,
# splitters, buckets sorted in LDS); the team's radix passes remain for
# grouped input, for the comparison flag and as the fallback of a call whose
# buckets outgrow the LDS.

def test_plan_names_the_sample_sort():
    g = _g()
    for n in (16385, 65536, 131072):
        assert g.debug_plan(n)["sample_sort"] == 1, n
    for n in (1, 16384, 131073):
        assert g.debug_plan(n)["sample_sort"] == 0, n
    # grouped input: the team's passes (its checkers sort the images)
    for n in (1, 16385, 64000, 131072):
        assert g.debug_plan(n, 16, True)["sample_sort"] == 0, n


@pytest.mark.parametrize("cfg,seed", [(5, 0), (5, 1), (5, 6)])
def test_sample_sort_vs_radix_team_vs_oracle(cfg, seed):
    w = workloads.config(cfg, seed)
    dev = device()
    note("sample vs radix team sort cfg=%d seed=%d" % (cfg, seed))
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold)
    b, s = to_dev(w.boxes, dev), to_dev(w.scores, dev)
    np.testing.assert_array_equal(_g().nms(b, s, w.iou_threshold).cpu().numpy(), want)
    np.testing.assert_array_equal(
        _g().nms(b, s, w.iou_threshold, radix_sort=True).cpu().numpy(), want)


@pytest.mark.parametrize("n", [16385, 40000, 65536, 131072])
def test_sample_sort_sorted_and_reversed_inputs(n):
    # already in order, in reverse order, and one score for all but a few
    dev = device()
    rng = np.random.default_rng(n)
    base = np.sort(rng.random(n).astype(np.float32))
    for name, scores in (("ascending", base), ("descending", base[::-1].copy()),
                         ("few_distinct", np.where(rng.random(n) < 0.001, rng.random(n),
                                                   0.5).astype(np.float32))):
        note("sample sort %s n=%d" % (name, n))
        order, _ = _g().debug_order(to_dev(scores, dev))
        np.testing.assert_array_equal(order.cpu().numpy(), np.argsort(-scores, kind="stable"),
                                      err_msg=name)


def test_sample_sort_fallback_when_a_bucket_overflows():
    # One box in 16 scores high (a set that holds every box the sort samples:
    # every 128th at 65,536 boxes) and every other box shares one low score:
    # all splitters fall among the high boxes and the last bucket takes the
    # low ones, more than one workgroup sorts in LDS.  The call runs again
    # with the radix passes; the result must not change.
    g = _g()
    dev = device()
    n = 65536
    rng = np.random.default_rng(17)
    scores = np.full(n, 0.125, np.float32)
    scores[::16] = (0.5 + 0.5 * rng.random(n // 16)).astype(np.float32)
    note("sample sort fallback n=%d" % n)
    order, _ = g.debug_order(to_dev(scores, dev))
    np.testing.assert_array_equal(order.cpu().numpy(), np.argsort(-scores, kind="stable"))
    w = workloads.config(5, 3)
    w = workloads.Workload("fallback", w.boxes, scores, w.iou_threshold)
    np.testing.assert_array_equal(_nms(w, False), oracle.c_nms(w.boxes, w.scores,
                                                                 w.iou_threshold))


@pytest.mark.parametrize("sizes", [[4096] * 5, [4097, 4096, 9000], [0, 20000], [1] * 17000])
def test_grouped_image_limits_end_to_end(sizes):
    # every image within the checkers' LDS sort (5 x 4096), an image above
    # it (the team runs the class and image passes too), an empty image
    # beside a large one, and more images than the LDS holds offsets for
    dev = device()
    n = int(sum(sizes))
    rng = np.random.default_rng(n + len(sizes))
    scores = _tied_scores(n, n + 7)
    cls = rng.integers(0, 50, n).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    note("grouped image limits, %d images, n=%d" % (len(sizes), n))
    order, sorder = _g().debug_order(to_dev(scores, dev), to_dev(cls, dev), to_dev(offs, dev))
    want, swant = _grouped_want(scores, cls, offs)
    np.testing.assert_array_equal(order.cpu().numpy(), want)
    np.testing.assert_array_equal(sorder.cpu().numpy(), swant)
    base = workloads.random_small(900 + len(sizes), n, canvas=400.0, score_levels=9, classes=6)
    w = workloads.Workload("grouped_limits", base.boxes, base.scores, 0.5, cls, offs)
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    np.testing.assert_array_equal(_nms(w, False), want)
