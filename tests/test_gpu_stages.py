"""Stage-level checks of the HIP path through the C ABI's test exports, plus
the race and state checks of the LeetCUDA page (bugs 1 and 2): repeated runs
must be identical, and the result must not depend on what the workspace held
before the call."""
import numpy as np
import torch
import pytest

import oracle
import workloads
from golden_cases import load_raw
from gpu_util import device, gpu_nms, note, to_dev

pytestmark = pytest.mark.gpu


def _g():
    import greedy_iou_nms_amd as g
    return g


# ---------------------------------------------------------------- sort

# ranking sort up to 16384 (one workgroup per 64 boxes; sizes around the
# 64-box chunks), radix passes over tiles of 4096 from 16385
@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 100, 1024, 1025, 2048, 2049, 4096, 4097, 8191,
                               8192, 8193, 16383, 16384, 16385, 65536])
def test_sort_order_is_stable_descending(n):
    dev = device()
    rng = np.random.default_rng(n)
    scores = (rng.integers(-8, 8, n) / 4).astype(np.float32)
    scores[rng.integers(0, n, max(1, n // 10))] = -0.0
    scores[rng.integers(0, n, max(1, n // 10))] = rng.random(max(1, n // 10)).astype(np.float32)
    note("sort n=%d" % n)
    order, sorder = _g().debug_order(to_dev(scores, dev))
    want = np.argsort(-scores, kind="stable")
    np.testing.assert_array_equal(order.cpu().numpy(), want)
    np.testing.assert_array_equal(sorder.cpu().numpy(), want)


@pytest.mark.parametrize("n", [100, 1000, 8192, 16384, 16385])
def test_sort_with_nan_scores_reports_and_still_permutes(n):
    # A NaN score is an error, but the kernels after the sort index memory
    # with the sorted order, so it must still be a permutation of 0 .. n-1.
    import ctypes
    g = _g()
    dev = device()
    rng = np.random.default_rng(7 + n)
    scores = rng.random(n).astype(np.float32)
    scores[rng.integers(0, n, max(1, n // 20))] = np.nan
    scores[rng.integers(0, n, max(1, n // 20))] = -np.inf
    scores[rng.integers(0, n, max(1, n // 50))] = np.float32(-np.nan)
    s = to_dev(scores, dev)
    note("sort with NaN n=%d" % n)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        buf = torch.empty(g.workspace_size(n, 0, False), dtype=torch.uint8, device=dev)
        order = torch.full((n,), -1, dtype=torch.int32, device=dev)
        st = g._lib.nms_debug_order(g._ptr(s), n, None, None, 0, g._ptr(order), None,
                                    g._ptr(buf), buf.numel(), ctypes.c_void_p(stream))
        torch.cuda.synchronize(dev)
    assert st == 3  # NMS_NONFINITE_INPUT
    np.testing.assert_array_equal(np.sort(order.cpu().numpy()), np.arange(n))


def test_sort_order_extreme_scores():
    dev = device()
    vals = np.float32([np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45, -1e-45, 0.0, -0.0, 1.0, -1.0])
    scores = np.tile(vals, 50)
    order, _ = _g().debug_order(to_dev(scores, dev))
    np.testing.assert_array_equal(order.cpu().numpy(), np.argsort(-scores, kind="stable"))


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_order(seed):
    dev = device()
    w = workloads.config(4, seed)
    note("grouped order seed=%d" % seed)
    order, sorder = _g().debug_order(to_dev(w.scores, dev), to_dev(w.class_ids, dev),
                                     to_dev(w.batch_offsets, dev))
    img, cls = oracle.groups_of(w.n, w.class_ids, w.batch_offsets)
    want = np.lexsort((np.arange(w.n), -w.scores, cls, img))
    np.testing.assert_array_equal(order.cpu().numpy(), want)
    np.testing.assert_array_equal(sorder.cpu().numpy(), np.argsort(-w.scores, kind="stable"))


# ---------------------------------------------------------------- mask

def _dense_mask(w):
    dev = device()
    m, order = _g().debug_mask(to_dev(w.boxes, dev), to_dev(w.scores, dev), w.iou_threshold,
                               to_dev(w.class_ids, dev), to_dev(w.batch_offsets, dev))
    return m.cpu().numpy().view(np.uint64), order.cpu().numpy()


@pytest.mark.parametrize("n", [1, 63, 64, 65, 127, 128, 129, 1000, 2100])
def test_mask_rows_match_definition(n):
    w = workloads.random_small(300 + n, n, canvas=5.0 * np.sqrt(n) + 20, score_levels=8)
    note("mask n=%d" % n)
    m, order = _dense_mask(w)
    np.testing.assert_array_equal(order, oracle.stable_order(w.scores))
    want = oracle.mask_rows(w.boxes, w.iou_threshold, order)
    assert m.shape == want.shape
    bad = np.argwhere(m != want)
    assert bad.size == 0, "first differing (row, word): %s" % (bad[:5].tolist(),)


def test_mask_layout_fixture():
    d = load_raw("layout_box5")
    w = workloads.Workload("layout", np.float32(d["boxes"]), np.float32(d["scores"]),
                           d["iou_threshold"])
    m, order = _dense_mask(w)
    for row, word, val in d["expected_mask_words"]:
        assert int(m[row, word]) == int(val, 16), (row, word)


def test_mask_rows_grouped():
    w = workloads.random_small(41, 700, canvas=120.0, score_levels=8, classes=3, images=4)
    m, order = _dense_mask(w)
    img, cls = oracle.groups_of(w.n, w.class_ids, w.batch_offsets)
    group = img * 1000 + cls
    np.testing.assert_array_equal(order, np.lexsort((np.arange(w.n), -w.scores, cls, img)))
    want = oracle.mask_rows(w.boxes, w.iou_threshold, order, group)
    assert np.array_equal(m, want)


# ---------------------------------------------------------------- threshold test

def _pairs_near(t, count, rng):
    t32 = np.float32(t)
    uni = np.exp(rng.uniform(np.log(1e-3), np.log(1e7), count)).astype(np.float32)
    base = (uni.astype(np.float64) * float(t32)).astype(np.float32)
    steps = rng.integers(-3, 4, count)
    inter = base.copy()
    for s in range(1, 4):
        inter = np.where(steps >= s, np.nextafter(inter, np.float32(np.inf)), inter)
        inter = np.where(steps <= -s, np.nextafter(inter, np.float32(0)), inter)
    inter = np.minimum(inter, uni).astype(np.float32)
    inter = np.maximum(inter, np.float32(0))
    return inter, uni


@pytest.mark.parametrize("t", [0.5, 0.7, 0.45, 0.3, 0.9, 1.0, 1e-20, 0.699999988079071,
                               0.5000000596046448])
def test_division_free_test_equals_float32_division(t):
    dev = device()
    rng = np.random.default_rng(int(t * 1e6) % 1000)
    inter, uni = _pairs_near(t, 2_000_000, rng)
    note("decide t=%r" % t)
    got = _g().debug_decide(to_dev(inter, dev), to_dev(uni, dev), t, True).cpu().numpy()
    with np.errstate(all="ignore"):
        want = (inter / uni) > np.float32(t)
    assert np.array_equal(got.astype(bool), want), int(np.sum(got.astype(bool) != want))


def test_literal_division_path_on_special_values():
    dev = device()
    vals = np.float32([0.0, -0.0, 1.0, -1.0, 0.5, 2.0, np.inf, -np.inf, np.nan, 1e-45, 3e38])
    inter = np.repeat(vals, vals.size)
    uni = np.tile(vals, vals.size)
    for t in (0.5, -0.5, 0.0):
        got = _g().debug_decide(to_dev(inter, dev), to_dev(uni, dev), t, False).cpu().numpy()
        with np.errstate(all="ignore"):
            want = (inter / uni) > np.float32(t)
        assert np.array_equal(got.astype(bool), want)


# ---------------------------------------------------------------- races and state

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_ten_runs_identical(cfg):
    w = workloads.config(cfg, 0)
    note("determinism cfg=%d" % cfg)
    first = gpu_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    for _ in range(9):
        again = gpu_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
        assert np.array_equal(first, again)


@pytest.mark.parametrize("cfg,runs", [(2, 300), (3, 100), (5, 100)])
def test_many_runs_match_oracle(cfg, runs):
    # A sweep build whose register use reached the 256-VGPR limit kept a
    # wrong box in about 5 % of the calls on the clustered 8192-box case:
    # every one of many calls must equal the oracle, not just the first.
    g = _g()
    dev = device()
    torch = pytest.importorskip("torch")
    w = workloads.config(cfg, 0)
    note("repeated runs cfg=%d x%d" % (cfg, runs))
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
    b = torch.from_numpy(w.boxes).to(dev)
    s = torch.from_numpy(w.scores).to(dev)
    ws = g.Workspace(dev)
    bad = []
    for it in range(runs):
        got = g.nms(b, s, w.iou_threshold, workspace=ws).cpu().numpy()
        if not np.array_equal(got, want):
            bad.append(it)
    assert not bad, "%d of %d calls differ from the oracle (first: call %d)" % (
        len(bad), runs, bad[0])


@pytest.mark.parametrize("fill", [0xFF, 0x00, "random"])
def test_workspace_contents_do_not_matter(fill):
    g = _g()
    dev = device()
    torch = pytest.importorskip("torch")
    for cfg in (1, 4):
        w = workloads.config(cfg, 1)
        want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets)
        ws = g.Workspace(dev)
        nbytes = g.workspace_size(w.n, 0 if w.batch_offsets is None else len(w.batch_offsets) - 1,
                                  w.class_ids is not None)
        buf = ws.get(nbytes, dev)
        if fill == "random":
            buf.copy_(torch.randint(0, 256, buf.shape, dtype=torch.uint8, device=dev))
        else:
            buf.fill_(fill)
        got = gpu_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids, w.batch_offsets,
                      workspace=ws)
        np.testing.assert_array_equal(got, want)


def test_reused_workspace_after_larger_call():
    g = _g()
    dev = device()
    ws = g.Workspace(dev)
    big = workloads.config(2, 0)
    small = workloads.config(1, 2)
    gpu_nms(big.boxes, big.scores, big.iou_threshold, workspace=ws)
    got = gpu_nms(small.boxes, small.scores, small.iou_threshold, workspace=ws)
    np.testing.assert_array_equal(got, oracle.c_nms(small.boxes, small.scores,
                                                    small.iou_threshold))


# ---------------------------------------------------------------- device-side errors

def test_device_detected_errors():
    g = _g()
    w = workloads.config(1, 0)
    s = w.scores.copy()
    s[17] = np.nan
    with pytest.raises(g.NMSError) as e:
        gpu_nms(w.boxes, s, 0.5)
    assert e.value.status == "NMS_NONFINITE_INPUT"
    b = w.boxes.copy()
    b[1000, 3] = np.inf
    with pytest.raises(g.NMSError) as e:
        gpu_nms(b, w.scores, 0.5)
    assert e.value.status == "NMS_NONFINITE_INPUT"
    for offs in ([0, 600, 500, 1024], [0, 512, 1000], [1, 512, 1024]):
        with pytest.raises(g.NMSError) as e:
            gpu_nms(w.boxes, w.scores, 0.5, None, np.array(offs, np.int64))
        assert e.value.status == "NMS_BAD_OFFSETS"
    # and the next call on the same device is unaffected
    np.testing.assert_array_equal(gpu_nms(w.boxes, w.scores, 0.5),
                                  oracle.c_nms(w.boxes, w.scores, 0.5))


def test_empty_and_single():
    torch = pytest.importorskip("torch")
    g = _g()
    dev = device()
    keep = g.nms(torch.zeros((0, 4), device=dev), torch.zeros((0,), device=dev), 0.5)
    assert keep.numel() == 0 and keep.dtype == torch.int64 and keep.device == dev
    keep = g.nms(torch.tensor([[0., 0., 1., 1.]], device=dev), torch.tensor([0.3], device=dev),
                 0.5)
    assert keep.cpu().tolist() == [0]
