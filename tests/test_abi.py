"""C-ABI checks that need no GPU: the library loads, exports every entry
point the public header declares, sizes workspaces from n alone, and rejects
bad arguments on the host before any device work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "greedy_nms.h")
LIB = os.path.join(ROOT, "greedy_iou_nms_amd", "libgreedy_nms.so")


def _lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    lib = ctypes.CDLL(LIB)
    lib.nms_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.nms_status_string.restype = ctypes.c_char_p
    lib.nms_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                            ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p, ctypes.c_size_t,
                            ctypes.c_void_p]
    return lib


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:nms_status|const char\s*\*)\s*(nms_\w+)\s*\(", text,
                                 re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ("nms_f32", "nms_f32_ex", "nms_workspace_size", "nms_status_string",
                 "nms_f32_profiled",
                 "nms_debug_order", "nms_debug_mask", "nms_debug_decide",
                 "nms_matrix_workspace_size", "nms_matrix_f32", "nms_matrix_f32_profiled"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


STATUS = {0: "NMS_OK", 1: "NMS_INVALID_ARG", 2: "NMS_WORKSPACE_TOO_SMALL",
          3: "NMS_NONFINITE_INPUT", 4: "NMS_BAD_OFFSETS", 5: "NMS_TOO_LARGE",
          6: "NMS_HIP_ERROR", 7: "NMS_BAD_BOXES"}


def test_status_strings():
    lib = _lib()
    for code, name in STATUS.items():
        assert lib.nms_status_string(code).decode() == name
    assert lib.nms_status_string(99).decode() == "NMS_UNKNOWN_STATUS"


def _ws(lib, n):
    out = ctypes.c_size_t(0)
    st = lib.nms_workspace_size(n, 0, 0, ctypes.byref(out))
    return st, out.value


def test_workspace_size_bound():
    lib = _lib()
    assert _ws(lib, 0) == (0, _ws(lib, 0)[1])
    prev = 0
    for n in (1, 63, 64, 65, 1000, 8192, 65536):
        st, b = _ws(lib, n)
        assert st == 0
        words = (n + 63) // 64
        mask = n * (((words + 15) // 16) * 16) * 8
        # dense mask + O(n) scratch (sort buffers, sorted boxes, row lists,
        # the per-box arrays of Matrix NMS) + the one-launch sort's words:
        # per team member (one per 1024 boxes, at most 32) 12 x 256 counts
        # and prefixes, 12 x 256 per-pass counts and 9 slots of 16 words,
        # plus 12 x 256 totals, 8 bytes each; its pass buffers hold three
        # times two 8-byte words per box (48 n bytes)
        members = min(32, (n + 1023) // 1024)
        team = 8 * (members * (2 * 12 * 256 + 12 * 256 + 9 * 16) + 12 * 256) + 48 * 64 * (
            (n + 63) // 64)
        assert mask <= b <= mask + 576 * n + 128 * 1024 + team
        assert b >= prev
        prev = b
    st, b = _ws(lib, 65536)
    assert b >= 512 * 1024 * 1024        # the dense N x N/64 bitmask dominates
    assert _ws(lib, -1)[0] == 1
    assert _ws(lib, 512001)[0] == 5
    assert _ws(lib, 512000)[0] == 0
    assert lib.nms_workspace_size(10, 0, 0, None) == 1


FAKE = 0x10000      # never dereferenced: every call below fails its host checks


def _call(lib, n, t=0.5, boxes=FAKE, scores=FAKE, cls=None, offs=None, num_images=0,
          keep=FAKE, ws=FAKE, ws_bytes=1 << 40, count=True):
    c = ctypes.c_int64(-7)
    st = lib.nms_f32(boxes, scores, n, t, cls, offs, num_images, keep,
                     ctypes.byref(c) if count else None, ws, ws_bytes, None)
    return STATUS[st], c.value


def test_host_argument_checks():
    lib = _lib()
    assert _call(lib, 0) == ("NMS_OK", 0)
    assert _call(lib, 0, boxes=None, scores=None, keep=None, ws=None) == ("NMS_OK", 0)
    assert _call(lib, -1)[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, t=float("nan"))[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, boxes=None)[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, scores=None)[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, keep=None)[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, ws=None)[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, count=False)[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, boxes=FAKE + 4)[0] == "NMS_INVALID_ARG"      # misaligned boxes
    assert _call(lib, 5, ws=FAKE + 64)[0] == "NMS_INVALID_ARG"        # misaligned workspace
    assert _call(lib, 5, num_images=3)[0] == "NMS_INVALID_ARG"        # images without offsets
    assert _call(lib, 5, offs=FAKE, num_images=0)[0] == "NMS_INVALID_ARG"
    assert _call(lib, 5, ws_bytes=100)[0] == "NMS_WORKSPACE_TOO_SMALL"
    assert _call(lib, 512001)[0] == "NMS_TOO_LARGE"
    # a failing call reports zero kept boxes
    assert _call(lib, 5, ws_bytes=100)[1] == 0


# ---------------------------------------------------------------- Matrix NMS

def _mlib():
    lib = _lib()
    c_i64, c_f, c_vp, c_sz = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    lib.nms_matrix_workspace_size.argtypes = [c_i64, ctypes.POINTER(c_sz)]
    lib.nms_matrix_workspace_size.restype = ctypes.c_int
    lib.nms_matrix_f32.argtypes = [c_vp, c_vp, c_i64, c_f, ctypes.c_double, c_vp,
                                   ctypes.POINTER(ctypes.c_int64), c_vp, c_sz, c_vp]
    lib.nms_matrix_f32.restype = ctypes.c_int
    return lib


def _mws(lib, n):
    out = ctypes.c_size_t(0)
    st = lib.nms_matrix_workspace_size(n, ctypes.byref(out))
    return st, out.value


def test_matrix_workspace_is_linear_and_below_greedy():
    lib = _mlib()
    for n in (1, 1000, 65536, 512000):
        st, b = _mws(lib, n)
        assert st == 0 and b < _ws(lib, n)[1]
        # no pairwise matrix: a few hundred bytes per box at most, plus the
        # one-launch sort's pass buffers (48 bytes per box) and its words
        # (under 2.5 MB)
        assert b <= (576 + 48) * n + (1 << 20) + (5 << 19)
    assert _mws(lib, 512001)[0] == 5
    assert lib.nms_matrix_workspace_size(5, None) == 1


def _mcall(lib, n, boxes=FAKE, scores=FAKE, t=0.1, sigma=0.5, keep=FAKE, count=True, ws=FAKE,
           ws_bytes=1 << 40):
    c = ctypes.c_int64(-1)
    st = lib.nms_matrix_f32(boxes, scores, n, t, sigma, keep, ctypes.byref(c) if count else None,
                            ws, ws_bytes, None)
    return STATUS[st], c.value


def test_matrix_host_argument_checks():
    lib = _mlib()
    assert _mcall(lib, 0) == ("NMS_OK", 0)
    assert _mcall(lib, -1)[0] == "NMS_INVALID_ARG"
    assert _mcall(lib, 5, t=float("nan"))[0] == "NMS_INVALID_ARG"
    for bad_sigma in (0.0, -1.0, float("nan"), float("inf")):
        assert _mcall(lib, 5, sigma=bad_sigma)[0] == "NMS_INVALID_ARG"
    assert _mcall(lib, 5, boxes=None)[0] == "NMS_INVALID_ARG"
    assert _mcall(lib, 5, keep=None)[0] == "NMS_INVALID_ARG"
    assert _mcall(lib, 5, count=False)[0] == "NMS_INVALID_ARG"
    assert _mcall(lib, 5, boxes=FAKE + 4)[0] == "NMS_INVALID_ARG"
    assert _mcall(lib, 5, ws=FAKE + 64)[0] == "NMS_INVALID_ARG"
    assert _mcall(lib, 5, ws_bytes=100) == ("NMS_WORKSPACE_TOO_SMALL", 0)
    assert _mcall(lib, 512001)[0] == "NMS_TOO_LARGE"


def test_binding_rejects_unusable_output_buffers():
    """The binding hands `out` to the library as a raw int64 pointer: a
    tensor of another dtype, a strided view, a tensor on another device or
    one too small for n boxes must be refused before any device work."""
    import torch

    import greedy_iou_nms_amd as g

    dev = torch.device("cpu")   # the check itself needs no GPU
    good = torch.empty(10, dtype=torch.int64)
    assert g._check_out(good, 10, dev) is good
    assert g._check_out(None, 10, dev).dtype == torch.int64
    with pytest.raises(TypeError):
        g._check_out(torch.empty(10, dtype=torch.int32), 10, dev)
    with pytest.raises(TypeError):
        g._check_out(torch.empty(20, dtype=torch.float32), 10, dev)
    with pytest.raises(ValueError):
        g._check_out(torch.empty(20, dtype=torch.int64)[::2], 10, dev)
    with pytest.raises(ValueError):
        g._check_out(torch.empty(9, dtype=torch.int64), 10, dev)
    with pytest.raises(ValueError):
        g._check_out(good, 10, torch.device("meta"))
    with pytest.raises(TypeError):
        g._check_out([0] * 10, 10, dev)
