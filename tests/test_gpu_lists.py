"""One image without the dense suppression bitmask: nms_f32 runs on a
workspace of nms_workspace_size_lists() bytes (the lists of nonzero mask
words, no dense rows), must not write past it, and must give the oracle's
result; an input dense enough to overflow a row tile's list returns
NMS_WORKSPACE_TOO_SMALL on that workspace and the oracle's result on one of
nms_workspace_size() bytes (the call runs again with dense rows).  The
binding grows its workspace by itself.

The lists are the page's "blocked bitmask" next step for the mask's memory
("LeetCUDA 14-nms", measured results)."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import device, note, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GUARD = 4 << 20
PATTERN = 0xAB
WORKSPACE_TOO_SMALL = 2


def _g():
    import greedy_iou_nms_amd as g
    return g


def _sizes(n):
    g = _g()
    lists = ctypes.c_size_t(0)
    full = ctypes.c_size_t(0)
    assert g._lib.nms_workspace_size_lists(n, ctypes.byref(lists)) == 0
    assert g._lib.nms_workspace_size(n, 0, 0, ctypes.byref(full)) == 0
    return lists.value, full.value


def _c_nms(w, ws_bytes, dev):
    """nms_f32 through the C ABI on a workspace of ws_bytes followed by a
    guard region filled with PATTERN; returns (status, kept, guard intact)."""
    g = _g()
    b = to_dev(w.boxes, dev)
    s = to_dev(w.scores, dev)
    ws = torch.full((ws_bytes + GUARD,), PATTERN, dtype=torch.uint8, device=dev)
    out = torch.empty(w.n, dtype=torch.int64, device=dev)
    count = ctypes.c_int64(0)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = g._lib.nms_f32(ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(s.data_ptr()), w.n,
                        ctypes.c_float(w.iou_threshold), None, None, 0,
                        ctypes.c_void_p(out.data_ptr()), ctypes.byref(count),
                        ctypes.c_void_p(ws.data_ptr()), ws_bytes, ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    guard_ok = bool(torch.all(ws[ws_bytes:] == PATTERN).item())
    return st, out[:count.value].cpu().numpy(), guard_ok


def _dense(n, seed, spread=1.0):
    # nearly equal boxes: every pair overlaps, every row tile's list overflows
    rng = np.random.default_rng(seed)
    base = np.array([100.0, 100.0, 200.0, 180.0])
    boxes = (base[None, :] + rng.uniform(-spread, spread, (n, 4))).astype(np.float32)
    return workloads.Workload("dense_%d" % n, boxes, rng.random(n).astype(np.float32), 0.5)


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_list_workspace_gives_the_oracle_result_and_stays_inside(cfg):
    dev = device()
    w = workloads.config(cfg, 0)
    lists, full = _sizes(w.n)
    assert lists < full
    note("list workspace cfg=%d n=%d (%d of %d bytes)" % (cfg, w.n, lists, full))
    st, got, guard_ok = _c_nms(w, lists, dev)
    assert st == 0
    assert guard_ok, "the call wrote past the list workspace"
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))


@pytest.mark.parametrize("n", [4096, 33000])
def test_dense_input_needs_the_full_workspace(n):
    # 4096: ranking sort and separate launches; 33000: the fused launch,
    # whose sweep gives up on the overflowing list and leaves it to the
    # plain sweep, which then asks for dense rows
    dev = device()
    w = _dense(n, 40 + n % 7)
    lists, full = _sizes(n)
    note("dense input n=%d on the list workspace" % n)
    st, _, guard_ok = _c_nms(w, lists, dev)
    assert st == WORKSPACE_TOO_SMALL
    assert guard_ok
    note("dense input n=%d on the full workspace" % n)
    st, got, guard_ok = _c_nms(w, full, dev)
    assert st == 0 and guard_ok
    want = oracle.c_nms(w.boxes, w.scores, w.iou_threshold)
    assert want.size < 8
    np.testing.assert_array_equal(got, want)


def test_binding_grows_its_workspace_for_dense_input():
    g = _g()
    dev = device()
    ws = g.Workspace(dev)
    small = workloads.config(1, 1)
    note("binding workspace: sparse then dense")
    got = g.nms(to_dev(small.boxes, dev), to_dev(small.scores, dev), small.iou_threshold,
                workspace=ws).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.c_nms(small.boxes, small.scores,
                                                    small.iou_threshold))
    lists, full = _sizes(4096)
    w = _dense(4096, 3)
    got = g.nms(to_dev(w.boxes, dev), to_dev(w.scores, dev), w.iou_threshold,
                workspace=ws).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.c_nms(w.boxes, w.scores, w.iou_threshold))
    assert ws.buf.numel() >= full
