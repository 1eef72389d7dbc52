"""Greedy IoU non-maximum suppression on MI355X (gfx950).

A thin ctypes binding over ``libgreedy_nms.so`` (C ABI in
``include/greedy_nms.h``).  Every step of the computation runs in the
library's HIP kernels; this module only checks tensor arguments, allocates the
output and the workspace with PyTorch, and passes pointers and the current
HIP stream.  There is no CPU fallback: importing fails loudly when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading
from typing import Dict, Optional, Tuple

import torch

__all__ = [
    "NMSError", "STAGES", "nms", "nms_profiled", "nms_static", "workspace_size", "Workspace",
    "debug_order", "debug_mask", "debug_decide", "debug_plan", "library_path",
    "MATRIX_STAGES", "matrix_nms", "matrix_nms_profiled", "matrix_workspace_size",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgreedy_nms.so")

STAGES = ("sort", "gather", "mask", "sweep", "compact")
MATRIX_STAGES = ("sort", "overlap_max", "decay")
_STATUS = {
    0: "NMS_OK", 1: "NMS_INVALID_ARG", 2: "NMS_WORKSPACE_TOO_SMALL",
    3: "NMS_NONFINITE_INPUT", 4: "NMS_BAD_OFFSETS", 5: "NMS_TOO_LARGE", 6: "NMS_HIP_ERROR",
    7: "NMS_BAD_BOXES",
}


class NMSError(RuntimeError):
    """A non-OK status from the library; ``status`` holds its name."""

    def __init__(self, status: str):
        super().__init__(status)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            "libgreedy_nms.so is not built (expected at %s); run "
            "`python -c 'import __graft_entry__ as g; g.build()'` from the repository root"
            % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    c_i64, c_f, c_vp, c_sz = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    p_i64 = ctypes.POINTER(ctypes.c_int64)
    lib.nms_workspace_size.argtypes = [c_i64, c_i64, ctypes.c_int, ctypes.POINTER(c_sz)]
    lib.nms_workspace_size.restype = ctypes.c_int
    lib.nms_workspace_size_lists.argtypes = [c_i64, ctypes.POINTER(c_sz)]
    lib.nms_workspace_size_lists.restype = ctypes.c_int
    common = [c_vp, c_vp, c_i64, c_f, c_vp, c_vp, c_i64, c_vp, p_i64, c_vp, c_sz, c_vp]
    lib.nms_f32.argtypes = common
    lib.nms_f32.restype = ctypes.c_int
    lib.nms_f32_ex.argtypes = common + [ctypes.c_int]
    lib.nms_f32_ex.restype = ctypes.c_int
    lib.nms_f32_profiled.argtypes = common + [ctypes.POINTER(ctypes.c_float), ctypes.c_int]
    lib.nms_f32_profiled.restype = ctypes.c_int
    lib.nms_f32_static.argtypes = [c_vp, c_vp, c_i64, c_f, c_vp, c_vp, c_i64, c_vp, p_i64, c_vp]
    lib.nms_f32_static.restype = ctypes.c_int
    lib.nms_status_string.argtypes = [ctypes.c_int]
    lib.nms_status_string.restype = ctypes.c_char_p
    lib.nms_debug_order.argtypes = [c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.nms_debug_order.restype = ctypes.c_int
    lib.nms_debug_mask.argtypes = [c_vp, c_vp, c_i64, c_f, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp,
                                   c_sz, c_vp]
    lib.nms_debug_mask.restype = ctypes.c_int
    lib.nms_debug_decide.argtypes = [c_vp, c_vp, c_i64, c_f, ctypes.c_int, c_vp, c_vp]
    lib.nms_debug_decide.restype = ctypes.c_int
    lib.nms_debug_plan.argtypes = [c_i64, c_i64, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)]
    lib.nms_debug_plan.restype = ctypes.c_int
    lib.nms_matrix_workspace_size.argtypes = [c_i64, ctypes.POINTER(c_sz)]
    lib.nms_matrix_workspace_size.restype = ctypes.c_int
    matrix = [c_vp, c_vp, c_i64, c_f, ctypes.c_double, c_vp, p_i64, c_vp, c_sz, c_vp]
    lib.nms_matrix_f32.argtypes = matrix
    lib.nms_matrix_f32.restype = ctypes.c_int
    lib.nms_matrix_f32_profiled.argtypes = matrix + [ctypes.POINTER(ctypes.c_float)]
    lib.nms_matrix_f32_profiled.restype = ctypes.c_int
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise NMSError(_STATUS.get(status, "NMS_UNKNOWN_%d" % status))


def workspace_size(n: int, num_images: int = 0, has_classes: bool = False) -> int:
    return _workspace_size(int(n), int(num_images), bool(has_classes))


@functools.lru_cache(maxsize=256)
def _workspace_size(n: int, num_images: int, has_classes: bool) -> int:
    # a bound from the sizes alone, so it can be remembered
    out = ctypes.c_size_t(0)
    _check(_lib.nms_workspace_size(n, num_images, int(has_classes), ctypes.byref(out)))
    return int(out.value)


@functools.lru_cache(maxsize=256)
def _workspace_size_lists(n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.nms_workspace_size_lists(n, ctypes.byref(out)))
    return int(out.value)


_WORKSPACE_TOO_SMALL = 2  # NMS_WORKSPACE_TOO_SMALL


def _raw_stream(device: torch.device) -> int:
    """The current stream of ``device`` as a raw hipStream_t value."""
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is not None:
        return int(get(device.index))
    return torch.cuda.current_stream(device).cuda_stream


class _OnDevice:
    """``torch.cuda.device(device)`` only when it is not already current (the
    switch costs a few microseconds per call)."""

    def __init__(self, device: torch.device):
        self.ctx = None if torch.cuda.current_device() == device.index else \
            torch.cuda.device(device)

    def __enter__(self):
        if self.ctx is not None:
            self.ctx.__enter__()

    def __exit__(self, *exc):
        if self.ctx is not None:
            return self.ctx.__exit__(*exc)
        return False


class Workspace:
    """Device scratch for the library, grown on demand and reused.  One
    Workspace must not serve two calls that may run concurrently."""

    def __init__(self, device=None):
        self.device = torch.device(device) if device is not None else None
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int, device: torch.device) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_tls = threading.local()


def _default_workspace(device: torch.device, stream: int) -> Workspace:
    cache = getattr(_tls, "ws", None)
    if cache is None:
        cache = _tls.ws = {}
    key = (device.index, stream)
    if key not in cache:
        cache[key] = Workspace(device)
    return cache[key]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_inputs(boxes, scores, class_ids, batch_offsets):
    if not (isinstance(boxes, torch.Tensor) and isinstance(scores, torch.Tensor)):
        raise TypeError("boxes and scores must be torch tensors")
    if not boxes.is_cuda:
        raise ValueError("boxes must be on a GPU device")
    if boxes.dtype != torch.float32 or scores.dtype != torch.float32:
        raise TypeError("boxes and scores must be float32")
    if boxes.dim() != 2 or boxes.shape[1] != 4:
        raise ValueError("boxes must have shape (N, 4)")
    n = boxes.shape[0]
    if scores.shape != (n,):
        raise ValueError("scores must have shape (N,)")
    if scores.device != boxes.device:
        raise ValueError("scores must be on the device of boxes")
    if not boxes.is_contiguous():
        boxes = boxes.contiguous()
    if not scores.is_contiguous():
        scores = scores.contiguous()
    if class_ids is not None:
        if class_ids.dtype != torch.int32 or class_ids.shape != (n,):
            raise TypeError("class_ids must be an int32 tensor of shape (N,)")
        if class_ids.device != boxes.device:
            raise ValueError("class_ids must be on the device of boxes")
        class_ids = class_ids.contiguous()
    num_images = 0
    if batch_offsets is not None:
        if batch_offsets.dtype != torch.int64 or batch_offsets.dim() != 1:
            raise TypeError("batch_offsets must be a 1-D int64 tensor")
        if batch_offsets.device != boxes.device:
            raise ValueError("batch_offsets must be on the device of boxes")
        batch_offsets = batch_offsets.contiguous()
        num_images = batch_offsets.shape[0] - 1
    return boxes, scores, class_ids, batch_offsets, num_images


PROFILE_NO_FUSION = 1  # nms_f32_profiled flag: mask and sweep as separate launches
PROFILE_ONE_LAUNCH = 2  # nms_f32_profiled flag: the one-launch path for small inputs
PROFILE_PASS_SORT = 4  # nms_f32_profiled flag: the radix sort as one launch per pass
PROFILE_RADIX_SORT = 8  # nms_f32_profiled flag: one image: radix passes, not sample sort
FLAG_ONE_LAUNCH = 1  # nms_f32_ex flag: the one-launch path for small inputs
FLAG_PASS_SORT = 2   # nms_f32_ex flag: the radix sort as one launch per pass
FLAG_RADIX_SORT = 4  # nms_f32_ex flag: one image: the team's radix passes, not sample sort


def _check_out(out: Optional[torch.Tensor], n: int, device: torch.device) -> torch.Tensor:
    """The output buffer: a fresh int64 tensor, or the caller's ``out``,
    which the library fills through a raw pointer with 8 bytes per kept box,
    so it must be a contiguous int64 tensor on ``device`` with room for n
    entries."""
    if out is None:
        return torch.empty(max(n, 1), dtype=torch.int64, device=device)
    if not isinstance(out, torch.Tensor):
        raise TypeError("out must be a torch tensor")
    if out.dtype != torch.int64:
        raise TypeError("out must be an int64 tensor (got %s)" % out.dtype)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if out.device != device:
        raise ValueError("out must be on the device of boxes (%s, got %s)" % (device, out.device))
    if out.numel() < n:
        raise ValueError("out holds %d entries; %d boxes need %d" % (out.numel(), n, n))
    return out


def _run(boxes, scores, iou_threshold, class_ids, batch_offsets, workspace, out, profiled,
         fuse=True, one_launch=False, pass_sort=False, radix_sort=False):
    boxes, scores, class_ids, batch_offsets, num_images = _check_inputs(
        boxes, scores, class_ids, batch_offsets)
    device = boxes.device
    n = boxes.shape[0]
    with _OnDevice(device):
        stream = _raw_stream(device)
        full = _workspace_size(n, num_images, class_ids is not None)
        # one image: the workspace without the dense bitmask first (enough
        # unless a row tile's list of nonzero words overflows; the library
        # then asks for the full size, see nms_workspace_size_lists)
        single = class_ids is None and num_images <= 1
        nbytes = _workspace_size_lists(n) if single else full
        ws = workspace if workspace is not None else _default_workspace(device, stream)
        out = _check_out(out, n, device)
        count = ctypes.c_int64(0)
        stage = (ctypes.c_float * len(STAGES))() if profiled else None
        flags = ((0 if fuse else PROFILE_NO_FUSION) | (PROFILE_ONE_LAUNCH if one_launch else 0) |
                 (PROFILE_PASS_SORT if pass_sort else 0) |
                 (PROFILE_RADIX_SORT if radix_sort else 0))
        ex_flags = ((FLAG_ONE_LAUNCH if one_launch else 0) | (FLAG_PASS_SORT if pass_sort else 0) |
                    (FLAG_RADIX_SORT if radix_sort else 0))

        def call(buf):
            args = [_ptr(boxes), _ptr(scores), n, ctypes.c_float(float(iou_threshold)),
                    _ptr(class_ids), _ptr(batch_offsets), num_images, _ptr(out),
                    ctypes.byref(count), _ptr(buf), buf.numel(), ctypes.c_void_p(stream)]
            if profiled:
                return _lib.nms_f32_profiled(*args, stage, flags)
            if ex_flags:
                return _lib.nms_f32_ex(*args, ex_flags)
            return _lib.nms_f32(*args)

        buf = ws.get(nbytes, device)
        status = call(buf)
        if status == _WORKSPACE_TOO_SMALL and buf.numel() < full:
            status = call(ws.get(full, device))
        _check(status)
    keep = out[:count.value]
    if profiled:
        return keep, {name: float(stage[i]) for i, name in enumerate(STAGES)}
    return keep


def nms(boxes: torch.Tensor, scores: torch.Tensor, iou_threshold: float,
        class_ids: Optional[torch.Tensor] = None, batch_offsets: Optional[torch.Tensor] = None,
        workspace: Optional[Workspace] = None, out: Optional[torch.Tensor] = None,
        one_launch: bool = False, pass_sort: bool = False,
        radix_sort: bool = False) -> torch.Tensor:
    """Greedy IoU NMS.  Returns the kept input indices (int64, on the boxes'
    device) in descending score order, ties by ascending index.  With
    ``class_ids`` and/or ``batch_offsets`` boxes suppress only boxes of the
    same (image, class); the result is one list in global score order.
    ``one_launch=True`` runs one image of at most 4096 boxes as a single
    launch (``nms_f32_ex`` with NMS_FLAG_ONE_LAUNCH); ``pass_sort=True``
    sorts with one launch per radix pass (NMS_FLAG_PASS_SORT);
    ``radix_sort=True`` sorts one image with the team's radix passes rather
    than by sample sort (NMS_FLAG_RADIX_SORT).  The result is the same
    either way."""
    return _run(boxes, scores, iou_threshold, class_ids, batch_offsets, workspace, out, False,
                True, one_launch, pass_sort, radix_sort)


STATIC_MAX_BOXES = 16384  # NMS_STATIC_MAX_BOXES


def nms_static(boxes: torch.Tensor, scores: torch.Tensor, iou_threshold: float,
               class_ids: Optional[torch.Tensor] = None,
               batch_offsets: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``nms`` through ``nms_f32_static``: the library's static scratch
    instead of a workspace (at most STATIC_MAX_BOXES boxes; calls that
    overlap on one device race).  With ``out`` given, the call allocates
    nothing on the device."""
    boxes, scores, class_ids, batch_offsets, num_images = _check_inputs(
        boxes, scores, class_ids, batch_offsets)
    device = boxes.device
    n = boxes.shape[0]
    with _OnDevice(device):
        stream = _raw_stream(device)
        out = _check_out(out, n, device)
        count = ctypes.c_int64(0)
        _check(_lib.nms_f32_static(_ptr(boxes), _ptr(scores), n,
                                   ctypes.c_float(float(iou_threshold)), _ptr(class_ids),
                                   _ptr(batch_offsets), num_images, _ptr(out),
                                   ctypes.byref(count), ctypes.c_void_p(stream)))
    return out[:count.value]


def nms_profiled(boxes, scores, iou_threshold, class_ids=None, batch_offsets=None,
                 workspace=None, out=None, fuse=True,
                 one_launch=False, pass_sort=False,
                 radix_sort=False) -> Tuple[torch.Tensor, Dict[str, float]]:
    """``nms`` plus per-stage GPU times in milliseconds (HIP events on the
    launch stream).  ``fuse=False`` runs the mask and the sweep as separate
    launches even where ``nms`` fuses them, so the mask kernel is timed
    alone; ``one_launch=True`` takes the one-launch path for small inputs
    (timed as the mask stage); ``pass_sort=True`` sorts with one launch per
    radix pass; ``radix_sort=True`` sorts one image with the team's radix
    passes rather than by sample sort."""
    if one_launch and not fuse:
        raise ValueError("one_launch and fuse=False exclude each other")
    return _run(boxes, scores, iou_threshold, class_ids, batch_offsets, workspace, out, True,
                fuse, one_launch, pass_sort, radix_sort)


def debug_order(scores: torch.Tensor, class_ids=None, batch_offsets=None):
    """The sort stage alone: (order, score_order) as int32 tensors."""
    n = scores.shape[0]
    dummy = torch.zeros((n, 4), dtype=torch.float32, device=scores.device)
    _, scores, class_ids, batch_offsets, num_images = _check_inputs(
        dummy, scores, class_ids, batch_offsets)
    device = scores.device
    with _OnDevice(device):
        stream = _raw_stream(device)
        buf = torch.empty(max(workspace_size(n, num_images, class_ids is not None), 256),
                          dtype=torch.uint8, device=device)
        order = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        sorder = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        _check(_lib.nms_debug_order(_ptr(scores), n, _ptr(class_ids), _ptr(batch_offsets),
                                    num_images, _ptr(order), _ptr(sorder), _ptr(buf),
                                    buf.numel(), ctypes.c_void_p(stream)))
    return order[:n], sorder[:n]


def debug_mask(boxes, scores, iou_threshold, class_ids=None, batch_offsets=None):
    """Sort, gather and the IoU mask, expanded to a dense (n, ceil(n/64))
    tensor of 64-bit words (returned as int64; view as uint64 on the CPU),
    together with the sorted order (int32) the rows refer to."""
    boxes, scores, class_ids, batch_offsets, num_images = _check_inputs(
        boxes, scores, class_ids, batch_offsets)
    n = boxes.shape[0]
    words = (n + 63) // 64
    device = boxes.device
    with _OnDevice(device):
        stream = _raw_stream(device)
        buf = torch.empty(max(workspace_size(n, num_images, class_ids is not None), 256),
                          dtype=torch.uint8, device=device)
        mask = torch.empty((max(n, 1), max(words, 1)), dtype=torch.int64, device=device)
        order = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        _check(_lib.nms_debug_mask(_ptr(boxes), _ptr(scores), n,
                                   ctypes.c_float(float(iou_threshold)), _ptr(class_ids),
                                   _ptr(batch_offsets), num_images, _ptr(mask), _ptr(order),
                                   _ptr(buf), buf.numel(), ctypes.c_void_p(stream)))
    return mask[:n, :words], order[:n]


PLAN_FIELDS = ("mask_qshift", "fused", "fused_qshift", "rank_sort", "small", "team_sort",
               "sample_sort")


def debug_plan(n: int, num_images: int = 0, has_classes: bool = False) -> Dict[str, int]:
    """The launch plan ``nms`` and ``debug_mask`` take for n boxes on the
    current device (see NMS_PLAN_* in include/greedy_nms.h)."""
    plan = (ctypes.c_int32 * 8)()
    _check(_lib.nms_debug_plan(int(n), int(num_images), int(bool(has_classes)), plan))
    return {name: int(plan[i]) for i, name in enumerate(PLAN_FIELDS)}


def debug_decide(inter: torch.Tensor, uni: torch.Tensor, iou_threshold: float,
                 positive_areas: bool) -> torch.Tensor:
    """The mask kernel's threshold test on given (intersection, union)
    pairs; returns uint8 (1 = suppress)."""
    if inter.dtype != torch.float32 or uni.dtype != torch.float32 or inter.shape != uni.shape:
        raise TypeError("inter and uni must be float32 tensors of one shape")
    inter = inter.contiguous()
    uni = uni.contiguous()
    out = torch.empty(inter.shape, dtype=torch.uint8, device=inter.device)
    with torch.cuda.device(inter.device):
        stream = torch.cuda.current_stream(inter.device).cuda_stream
        _check(_lib.nms_debug_decide(_ptr(inter), _ptr(uni), inter.numel(),
                                     ctypes.c_float(float(iou_threshold)),
                                     int(bool(positive_areas)), _ptr(out),
                                     ctypes.c_void_p(stream)))
    return out


# ---------------------------------------------------------------- Matrix NMS

def matrix_workspace_size(n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.nms_matrix_workspace_size(int(n), ctypes.byref(out)))
    return int(out.value)


def _run_matrix(boxes, scores, score_threshold, sigma, workspace, out, profiled):
    boxes, scores, _, _, _ = _check_inputs(boxes, scores, None, None)
    device = boxes.device
    n = boxes.shape[0]
    with _OnDevice(device):
        stream = _raw_stream(device)
        nbytes = matrix_workspace_size(n)
        ws = workspace if workspace is not None else _default_workspace(device, stream)
        buf = ws.get(nbytes, device)
        out = _check_out(out, n, device)
        count = ctypes.c_int64(0)
        args = [_ptr(boxes), _ptr(scores), n, ctypes.c_float(float(score_threshold)),
                ctypes.c_double(float(sigma)), _ptr(out), ctypes.byref(count), _ptr(buf),
                buf.numel(), ctypes.c_void_p(stream)]
        stage = None
        if profiled:
            stage = (ctypes.c_float * len(MATRIX_STAGES))()
            _check(_lib.nms_matrix_f32_profiled(*args, stage))
        else:
            _check(_lib.nms_matrix_f32(*args))
    keep = out[:count.value]
    if profiled:
        return keep, {name: float(stage[i]) for i, name in enumerate(MATRIX_STAGES)}
    return keep


def matrix_nms(boxes: torch.Tensor, scores: torch.Tensor, score_threshold: float,
               sigma: float = 0.5, workspace: Optional[Workspace] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Matrix NMS with the Gaussian decay (see include/greedy_nms.h): the kept
    input indices (int64, on the boxes' device) in descending score order."""
    return _run_matrix(boxes, scores, score_threshold, sigma, workspace, out, False)


def matrix_nms_profiled(boxes, scores, score_threshold, sigma=0.5, workspace=None, out=None):
    """``matrix_nms`` plus per-stage GPU times in milliseconds."""
    return _run_matrix(boxes, scores, score_threshold, sigma, workspace, out, True)
