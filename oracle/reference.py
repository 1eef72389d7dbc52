"""CPU oracle for greedy IoU NMS -- TEST INFRASTRUCTURE ONLY (see package doc).

Two independent implementations of the same definition live here:

* ``c_nms``: ctypes front-end of ``nms_oracle.c`` (plain C, single thread,
  float32 IEEE arithmetic built with ``-ffp-contract=off``).
* ``np_nms``: numpy float32, vectorised over one kept row at a time.

Both follow the greedy procedure of "LeetCUDA 14-nms" (introduction and the
"algorithm and data flow" steps): a stable descending score sort, then boxes
are visited in that order, a box not yet removed is kept and removes every
later box of its group whose IoU exceeds the threshold strictly, and the kept
boxes are returned as original input indices (that page's bug 3 fix).
Suppression only within equal class follows the class check of "YOLOv5
post-processing GPU port" (section 2.2); equal scores rank the lower input
index first (its priority rule in the same section, and the stable sort of the
LeetCUDA page).

``certify`` checks a kept list K against three properties that determine the
greedy result uniquely (by induction over sorted position):
  I1  K is strictly increasing in sorted position;
  I2  no two members i before j of one group have IoU(i, j) > t;
  I3  every non-member j has a member i before it, same group, IoU(i, j) > t.
``brute_force`` enumerates all subsets of a tiny input and returns the unique
one satisfying I2 and I3.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nms_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# The oracle's own status numbering (nms_oracle.c).
ORACLE_STATUS = {0: "OK", 1: "INVALID_ARG", 3: "NONFINITE_INPUT", 4: "BAD_OFFSETS",
                 5: "BAD_BOXES"}

C_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-mfpmath=sse",
           "-msse2", "-fPIC", "-shared"]


class OracleError(Exception):
    def __init__(self, status: str):
        super().__init__(status)
        self.status = status


def build_c_oracle(force: bool = False, src: str = _SRC, out: str = _LIB,
                   extra_flags=()) -> str:
    """Compile nms_oracle.c with gcc into a shared library (in-tree)."""
    if (not force and os.path.exists(out)
            and os.path.getmtime(out) >= os.path.getmtime(src)):
        return out
    cmd = ["gcc", *C_FLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib_cache = {}


def _load(path: str = _LIB):
    if path not in _lib_cache:
        if path == _LIB:
            build_c_oracle()
        lib = ctypes.CDLL(path)
        f = lib.oracle_nms
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        m = lib.oracle_matrix_nms
        m.restype = ctypes.c_int
        m.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                      ctypes.c_double, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                      ctypes.POINTER(ctypes.c_int64)]
        g = lib.oracle_pair_iou
        g.restype = None
        g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                      ctypes.c_void_p]
        _lib_cache[path] = lib
    return _lib_cache[path]


def _ptr(a):
    return None if a is None else a.ctypes.data


def c_nms(boxes, scores, iou_threshold, class_ids=None, batch_offsets=None,
          lib_path: str = _LIB, return_borderline: bool = False):
    """Run the C oracle. Returns the kept int64 indices (and the borderline
    pair count when asked); raises OracleError on a non-OK status."""
    boxes = np.ascontiguousarray(boxes, dtype=np.float32).reshape(-1, 4)
    scores = np.ascontiguousarray(scores, dtype=np.float32).reshape(-1)
    n = boxes.shape[0]
    if scores.shape[0] != n:
        raise OracleError("INVALID_ARG")
    cls = None if class_ids is None else np.ascontiguousarray(class_ids, dtype=np.int32)
    offs = None if batch_offsets is None else np.ascontiguousarray(batch_offsets, dtype=np.int64)
    num_images = 0 if offs is None else offs.shape[0] - 1
    keep = np.zeros(max(n, 1), dtype=np.int64)
    cnt = ctypes.c_int64(-1)
    border = ctypes.c_int64(0)
    lib = _load(lib_path)
    st = lib.oracle_nms(_ptr(boxes), _ptr(scores), n, ctypes.c_float(iou_threshold),
                        _ptr(cls), _ptr(offs), num_images, _ptr(keep), ctypes.byref(cnt),
                        ctypes.byref(border))
    if st != 0:
        raise OracleError(ORACLE_STATUS.get(st, "UNKNOWN_%d" % st))
    out = keep[:cnt.value].copy()
    return (out, border.value) if return_borderline else out


def c_matrix_nms(boxes, scores, score_threshold, sigma=0.5, lib_path: str = _LIB,
                 return_borderline: bool = False):
    """Matrix NMS (Gaussian decay) through the C oracle: kept int64 input
    indices in descending score order (and, when asked, the number of boxes
    decided within a relative 1e-9 of the threshold)."""
    boxes = np.ascontiguousarray(boxes, dtype=np.float32).reshape(-1, 4)
    scores = np.ascontiguousarray(scores, dtype=np.float32).reshape(-1)
    n = boxes.shape[0]
    if scores.shape[0] != n:
        raise OracleError("INVALID_ARG")
    keep = np.zeros(max(n, 1), dtype=np.int64)
    cnt = ctypes.c_int64(-1)
    border = ctypes.c_int64(0)
    st = _load(lib_path).oracle_matrix_nms(_ptr(boxes), _ptr(scores), n,
                                           ctypes.c_float(score_threshold), float(sigma),
                                           _ptr(keep), ctypes.byref(cnt), ctypes.byref(border))
    if st != 0:
        raise OracleError(ORACLE_STATUS.get(st, "UNKNOWN_%d" % st))
    out = keep[:cnt.value].copy()
    return (out, border.value) if return_borderline else out


def c_pair_iou(boxes, a, b, lib_path: str = _LIB):
    """float32 IoU of box pairs (a[k], b[k]) through the C oracle's expression."""
    boxes = np.ascontiguousarray(boxes, dtype=np.float32).reshape(-1, 4)
    a = np.ascontiguousarray(a, dtype=np.int64)
    b = np.ascontiguousarray(b, dtype=np.int64)
    out = np.empty(a.shape[0], dtype=np.float32)
    _load(lib_path).oracle_pair_iou(_ptr(boxes), _ptr(a), _ptr(b), a.shape[0], _ptr(out))
    return out


# ---------------------------------------------------------------------------
# numpy float32 implementation
# ---------------------------------------------------------------------------

def _validate(boxes, scores, t, class_ids, batch_offsets):
    n = boxes.shape[0]
    if scores.shape[0] != n or np.isnan(np.float32(t)):
        raise OracleError("INVALID_ARG")
    if class_ids is not None and class_ids.shape[0] != n:
        raise OracleError("INVALID_ARG")
    if batch_offsets is not None:
        o = batch_offsets
        if o.shape[0] < 2 or o[0] != 0 or o[-1] != n or np.any(np.diff(o) < 0):
            raise OracleError("BAD_OFFSETS")
    if np.any(np.isnan(scores)) or not np.all(np.isfinite(boxes)):
        raise OracleError("NONFINITE_INPUT")


def groups_of(n, class_ids=None, batch_offsets=None):
    """(image, class) of every box; a missing part is 0."""
    img = np.zeros(n, dtype=np.int64)
    if batch_offsets is not None:
        img = np.repeat(np.arange(batch_offsets.shape[0] - 1, dtype=np.int64),
                        np.diff(batch_offsets))
    cls = np.zeros(n, dtype=np.int64) if class_ids is None else class_ids.astype(np.int64)
    return img, cls


def stable_order(scores):
    """Indices by score descending; equal scores keep ascending index."""
    return np.argsort(-np.asarray(scores, dtype=np.float32), kind="stable").astype(np.int64)


def areas_f32(boxes):
    return (boxes[:, 2] - boxes[:, 0]) * (boxes[:, 3] - boxes[:, 1])


def iou_row_f32(bi, ai, bj, aj):
    """float32 IoU of one box (bi, area ai) against boxes bj (areas aj)."""
    zero = np.float32(0.0)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        xx1 = np.maximum(bi[0], bj[:, 0])
        yy1 = np.maximum(bi[1], bj[:, 1])
        xx2 = np.minimum(bi[2], bj[:, 2])
        yy2 = np.minimum(bi[3], bj[:, 3])
        w = np.maximum(xx2 - xx1, zero)
        h = np.maximum(yy2 - yy1, zero)
        inter = w * h
        uni = (ai + aj) - inter
        return inter / uni


def np_iou_pairs(boxes, a, b):
    boxes = np.asarray(boxes, dtype=np.float32).reshape(-1, 4)
    area = areas_f32(boxes)
    out = np.empty(len(a), dtype=np.float32)
    for k, (i, j) in enumerate(zip(a, b)):
        out[k] = iou_row_f32(boxes[i], area[i], boxes[j:j + 1], area[j:j + 1])[0]
    return out


def np_nms(boxes, scores, iou_threshold, class_ids=None, batch_offsets=None):
    """Greedy NMS in numpy float32 (independent of the C oracle)."""
    boxes = np.asarray(boxes, dtype=np.float32).reshape(-1, 4)
    scores = np.asarray(scores, dtype=np.float32).reshape(-1)
    cls_in = None if class_ids is None else np.asarray(class_ids, dtype=np.int32)
    offs = None if batch_offsets is None else np.asarray(batch_offsets, dtype=np.int64)
    _validate(boxes, scores, iou_threshold, cls_in, offs)
    n = boxes.shape[0]
    t = np.float32(iou_threshold)
    img, cls = groups_of(n, cls_in, offs)
    area = areas_f32(boxes)
    order = stable_order(scores)
    removed = np.zeros(n, dtype=bool)
    keep = []
    for p in range(n):
        i = order[p]
        if removed[i]:
            continue
        keep.append(i)
        rest = order[p + 1:]
        rest = rest[(~removed[rest]) & (img[rest] == img[i]) & (cls[rest] == cls[i])]
        if rest.size:
            iou = iou_row_f32(boxes[i], area[i], boxes[rest], area[rest])
            removed[rest[iou > t]] = True
    return np.asarray(keep, dtype=np.int64)


# ---------------------------------------------------------------------------
# certificate and brute force
# ---------------------------------------------------------------------------

def certify(boxes, scores, iou_threshold, keep, class_ids=None, batch_offsets=None):
    """Return None if ``keep`` is the greedy result, else a string saying
    which of I1/I2/I3 fails."""
    boxes = np.asarray(boxes, dtype=np.float32).reshape(-1, 4)
    scores = np.asarray(scores, dtype=np.float32).reshape(-1)
    keep = np.asarray(keep, dtype=np.int64)
    n = boxes.shape[0]
    t = np.float32(iou_threshold)
    cls_in = None if class_ids is None else np.asarray(class_ids, dtype=np.int32)
    offs = None if batch_offsets is None else np.asarray(batch_offsets, dtype=np.int64)
    img, cls = groups_of(n, cls_in, offs)
    if keep.size and (keep.min() < 0 or keep.max() >= n):
        return "I1: index out of range"
    if np.unique(keep).size != keep.size:
        return "I1: repeated index"
    order = stable_order(scores)
    pos = np.empty(n, dtype=np.int64)
    pos[order] = np.arange(n)
    kp = pos[keep]
    if np.any(np.diff(kp) <= 0):
        return "I1: not increasing in sorted position"
    area = areas_f32(boxes)
    in_k = np.zeros(n, dtype=bool)
    in_k[keep] = True
    covered = np.zeros(n, dtype=bool)
    for i in keep:
        later = order[pos[i] + 1:]
        later = later[(img[later] == img[i]) & (cls[later] == cls[i])]
        if later.size:
            hit = later[iou_row_f32(boxes[i], area[i], boxes[later], area[later]) > t]
            covered[hit] = True
    if np.any(covered & in_k):
        return "I2: a kept box overlaps an earlier kept box above the threshold"
    if np.any(~covered & ~in_k):
        return "I3: a removed box has no earlier kept box overlapping it"
    return None


def brute_force(boxes, scores, iou_threshold, class_ids=None, batch_offsets=None):
    """All subsets of a tiny input (n <= 14); returns the unique subset
    satisfying I2 and I3, in sorted-position order.  Raises if not unique."""
    boxes = np.asarray(boxes, dtype=np.float32).reshape(-1, 4)
    scores = np.asarray(scores, dtype=np.float32).reshape(-1)
    n = boxes.shape[0]
    assert n <= 14
    t = np.float32(iou_threshold)
    cls_in = None if class_ids is None else np.asarray(class_ids, dtype=np.int32)
    offs = None if batch_offsets is None else np.asarray(batch_offsets, dtype=np.int64)
    img, cls = groups_of(n, cls_in, offs)
    order = stable_order(scores)
    pos = np.empty(n, dtype=np.int64)
    pos[order] = np.arange(n)
    area = areas_f32(boxes)
    sup = np.zeros((n, n), dtype=bool)   # sup[i, j]: i precedes j and removes it
    for i in range(n):
        iou = iou_row_f32(boxes[i], area[i], boxes, area)
        sup[i] = (pos[i] < pos) & (img == img[i]) & (cls == cls[i]) & (iou > t)
    sup_mask = [int(sum(1 << j for j in range(n) if sup[i, j])) for i in range(n)]
    found = []
    for s in range(1 << n):
        ok = True
        cover = 0
        for i in range(n):
            if s >> i & 1:
                if sup_mask[i] & s:
                    ok = False
                    break
                cover |= sup_mask[i]
        if ok and (cover | s) == (1 << n) - 1:
            found.append(s)
    if len(found) != 1:
        raise AssertionError("expected exactly one fixpoint, found %d" % len(found))
    members = [i for i in range(n) if found[0] >> i & 1]
    return np.asarray(sorted(members, key=lambda i: pos[i]), dtype=np.int64)


# ---------------------------------------------------------------------------
# the suppression bitmask by definition
# ---------------------------------------------------------------------------

def mask_rows(boxes, iou_threshold, order, group=None):
    """Dense suppression bitmask for boxes visited in ``order``.

    Row p (sorted position p) has W = ceil(n/64) uint64 words; bit l of word c
    is 1 iff q = 64c + l satisfies p < q < n, group[order[q]] ==
    group[order[p]] (when ``group`` is given) and IoU(order[p], order[q]) > t.
    This is the layout of the "LeetCUDA 14-nms" Phase 1 bitmask (bit k of word
    w stands for box w*width + k in every row; boxes at or before the row never
    vote), with 64-bit words.
    """
    boxes = np.asarray(boxes, dtype=np.float32).reshape(-1, 4)
    order = np.asarray(order, dtype=np.int64)
    n = boxes.shape[0]
    w_words = (n + 63) // 64
    t = np.float32(iou_threshold)
    sb = boxes[order]
    sa = areas_f32(sb)
    g = None if group is None else np.asarray(group)[order]
    out = np.zeros((n, w_words), dtype=np.uint64)
    bits = np.zeros(w_words * 64, dtype=bool)
    for p in range(n):
        bits[:] = False
        if p + 1 < n:
            hit = iou_row_f32(sb[p], sa[p], sb[p + 1:], sa[p + 1:]) > t
            if g is not None:
                hit &= g[p + 1:] == g[p]
            bits[p + 1:n] = hit
        out[p] = np.packbits(bits, bitorder="little").view("<u8")
    return out


# ---------------------------------------------------------------------------
# Matrix NMS, the page's naive formulation
# ---------------------------------------------------------------------------

def np_matrix_nms(boxes, scores, score_threshold, sigma=0.5):
    """Matrix NMS with the Gaussian decay, following the naive steps listed on
    "Fastest Matrix NMS in the West (Part 2)" ("What do we need to compute?"):
    build the triangular IoU matrix (father p < child q, zero elsewhere),
    reduce it to the per-box maximum overlap with its own fathers, broadcast,
    build the whole decay matrix exp((omax_p^2 - O_pq^2) / sigma), reduce it
    to one decay per box (minimum over every p), multiply the scores and keep
    those >= the threshold.  float32 IoUs (0/0 counted as 0), binary64 decay.
    For non-negative scores this equals the C oracle's per-pair test; it is an
    independent second implementation for small inputs."""
    boxes = np.asarray(boxes, dtype=np.float32).reshape(-1, 4)
    scores = np.asarray(scores, dtype=np.float32).reshape(-1)
    n = boxes.shape[0]
    if scores.shape[0] != n or np.isnan(np.float32(score_threshold)) or not sigma > 0:
        raise OracleError("INVALID_ARG")
    if np.any(np.isnan(scores)) or not np.all(np.isfinite(boxes)):
        raise OracleError("NONFINITE_INPUT")
    if np.any(boxes[:, 0] > boxes[:, 2]) or np.any(boxes[:, 1] > boxes[:, 3]):
        raise OracleError("BAD_BOXES")
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    order = stable_order(scores)
    sb = boxes[order]
    s = scores[order].astype(np.float64)
    area = areas_f32(sb)
    O = np.zeros((n, n), dtype=np.float32)
    for p in range(n - 1):
        o = iou_row_f32(sb[p], area[p], sb[p + 1:], area[p + 1:])
        O[p, p + 1:] = np.where(np.isnan(o), np.float32(0.0), o)
    omax = O.max(axis=0).astype(np.float64)
    Od = O.astype(np.float64)
    decay = np.exp((omax[:, None] * omax[:, None] - Od * Od) / float(sigma))
    s_new = s * decay.min(axis=0)
    return order[s_new >= float(np.float32(score_threshold))]
