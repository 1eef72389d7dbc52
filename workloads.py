"""Seeded synthetic NMS workloads (boxes, scores, classes, batch offsets).

This module holds only random draws and box construction; it performs none of
the suppression arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it.

Every recipe draws with ``numpy.random.default_rng(seed)`` (PCG64), in float64,
in the order written below, and casts each coordinate to float32 at the end:
``x1 = float32(x1_64)``, ``x2 = float32(x1_64 + w_64)`` (and likewise for y).
Clustered boxes use ``x1_64 = cx - w/2``.  Nothing is clipped or shuffled.

The five named workloads stand in for detector outputs (boxes of a single
image, clustered duplicates, tie-heavy scores, a batch of images with 80
classes, and one large image); no dataset is read.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass
class Workload:
    name: str
    boxes: np.ndarray                  # (N, 4) float32, x1 y1 x2 y2
    scores: np.ndarray                 # (N,) float32
    iou_threshold: float
    class_ids: Optional[np.ndarray] = None     # (N,) int32 or None
    batch_offsets: Optional[np.ndarray] = None  # (num_images+1,) int64 or None
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.boxes.shape[0])

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.boxes, self.scores, self.class_ids, self.batch_offsets):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        h.update(np.float32(self.iou_threshold).tobytes())
        return h.hexdigest()


def _uniform_boxes(rng, n, canvas, wmin=8.0, wmax=120.0):
    """x1, y1 ~ U[0, canvas); w, h ~ U[wmin, wmax); drawn in that order."""
    x1 = rng.uniform(0.0, canvas, n)
    y1 = rng.uniform(0.0, canvas, n)
    w = rng.uniform(wmin, wmax, n)
    h = rng.uniform(wmin, wmax, n)
    return _pack(x1, y1, w, h)


def _clustered_boxes(rng, n, n_centres, canvas, jitter, assign):
    """Cluster centres ~ U[0,canvas)^2, per-cluster base w,h ~ U[30,90);
    box k belongs to cluster assign(k); centre jitter N(0, jitter) per axis;
    per-box size factor (1 + N(0, 0.1)) on w and h."""
    cx = rng.uniform(0.0, canvas, n_centres)
    cy = rng.uniform(0.0, canvas, n_centres)
    bw = rng.uniform(30.0, 90.0, n_centres)
    bh = rng.uniform(30.0, 90.0, n_centres)
    k = assign(np.arange(n))
    jx = rng.normal(0.0, jitter, n)
    jy = rng.normal(0.0, jitter, n)
    fw = 1.0 + rng.normal(0.0, 0.1, n)
    fh = 1.0 + rng.normal(0.0, 0.1, n)
    w = bw[k] * fw
    h = bh[k] * fh
    x1 = cx[k] + jx - w / 2.0
    y1 = cy[k] + jy - h / 2.0
    return _pack(x1, y1, w, h)


def _pack(x1, y1, w, h):
    out = np.empty((x1.shape[0], 4), dtype=np.float32)
    out[:, 0] = x1.astype(np.float32)
    out[:, 1] = y1.astype(np.float32)
    out[:, 2] = (x1 + w).astype(np.float32)
    out[:, 3] = (y1 + h).astype(np.float32)
    return out


def single_sparse(seed: int = 0, n: int = 1024) -> Workload:
    """Single image, N=1024: x1,y1 ~ U[0,1000), w,h ~ U[8,120);
    scores = rng.random() as float32; threshold 0.5."""
    rng = np.random.default_rng(seed)
    boxes = _uniform_boxes(rng, n, 1000.0)
    scores = rng.random(n).astype(np.float32)
    return Workload("single_sparse_n%d" % n, boxes, scores, 0.5,
                    meta={"seed": seed, "recipe": "uniform 1000^2"})


def single_clustered(seed: int = 0, n: int = 8192) -> Workload:
    """Single image, N=8192: 256 centres on [0,2000)^2, 32 boxes per cluster
    (box k -> cluster k // 32), jitter N(0,6); scores ~ Beta(2,5); threshold 0.5."""
    rng = np.random.default_rng(seed)
    per = 32
    boxes = _clustered_boxes(rng, n, n // per, 2000.0, 6.0, lambda k: k // per)
    scores = rng.beta(2.0, 5.0, n).astype(np.float32)
    return Workload("single_clustered_n%d" % n, boxes, scores, 0.5,
                    meta={"seed": seed, "recipe": "256 clusters x 32, 2000^2"})


def tie_stress(seed: int = 0, n: int = 4096) -> Workload:
    """N=4096 boxes with the N=1024 law on a [0,400) canvas (heavy overlap);
    scores = k/16 with k ~ U{1..16} (exact in float32); threshold 0.7."""
    rng = np.random.default_rng(seed)
    boxes = _uniform_boxes(rng, n, 400.0)
    scores = (rng.integers(1, 17, n).astype(np.float64) / 16.0).astype(np.float32)
    return Workload("tie_stress_n%d" % n, boxes, scores, 0.7,
                    meta={"seed": seed, "recipe": "uniform 400^2, 16 score levels"})


def batched_classes(seed: int = 0, images: int = 16, per_image: int = 4000,
                    classes: int = 80) -> Workload:
    """16 images x 4000 boxes on a 640x640 canvas: per image 64 centres,
    box k -> centre k mod 64, jitter N(0,6); class ~ U{0..79}; scores ~ U(0.25,1);
    suppression only within equal (image, class); threshold 0.45."""
    rng = np.random.default_rng(seed)
    bx, sc, cl = [], [], []
    for _ in range(images):
        bx.append(_clustered_boxes(rng, per_image, 64, 640.0, 6.0, lambda k: k % 64))
        cl.append(rng.integers(0, classes, per_image).astype(np.int32))
        sc.append(rng.uniform(0.25, 1.0, per_image).astype(np.float32))
    boxes = np.concatenate(bx)
    scores = np.concatenate(sc)
    class_ids = np.concatenate(cl)
    offsets = np.arange(images + 1, dtype=np.int64) * per_image
    return Workload("batched_%dx%d_c%d" % (images, per_image, classes), boxes, scores,
                    0.45, class_ids=class_ids, batch_offsets=offsets,
                    meta={"seed": seed, "recipe": "per-image 64 clusters, 640^2"})


def large_mixed(seed: int = 0, n: int = 65536) -> Workload:
    """N=65536: first half uniform (N=1024 law on [0,8192)); second half 2048
    centres on [0,8192)^2 with 16 boxes each (box k -> centre k // 16), jitter
    N(0,8), cluster sizes as in the clustered law; scores = rng.random();
    threshold 0.5."""
    rng = np.random.default_rng(seed)
    half = n // 2
    a = _uniform_boxes(rng, half, 8192.0)
    b = _clustered_boxes(rng, n - half, (n - half) // 16, 8192.0, 8.0, lambda k: k // 16)
    boxes = np.concatenate([a, b])
    scores = rng.random(n).astype(np.float32)
    return Workload("large_mixed_n%d" % n, boxes, scores, 0.5,
                    meta={"seed": seed, "recipe": "half uniform 8192^2, half 2048x16 clusters"})


CONFIGS = {
    1: single_sparse,
    2: single_clustered,
    3: tie_stress,
    4: batched_classes,
    5: large_mixed,
}


def config(idx: int, seed: int = 0) -> Workload:
    return CONFIGS[idx](seed=seed)


def random_small(seed: int, n: int, canvas: float = 100.0, score_levels: int = 0,
                 classes: int = 0, images: int = 0) -> Workload:
    """Small random case for cross-checks: uniform boxes of size U[4,40) on a
    ``canvas``-wide square; scores ``rng.random()`` or, with score_levels>0,
    k/score_levels (tie-heavy); optional classes and image split."""
    rng = np.random.default_rng(seed)
    boxes = _uniform_boxes(rng, n, canvas, 4.0, 40.0)
    if score_levels > 0:
        scores = (rng.integers(0, score_levels, n).astype(np.float64)
                  / score_levels).astype(np.float32)
    else:
        scores = rng.random(n).astype(np.float32)
    t = float(np.float32(rng.uniform(0.2, 0.8)))
    class_ids = rng.integers(0, classes, n).astype(np.int32) if classes > 0 else None
    offsets = None
    if images > 0:
        cuts = np.sort(rng.integers(0, n + 1, images - 1))
        offsets = np.concatenate([[0], cuts, [n]]).astype(np.int64)
    return Workload("random_small_s%d_n%d" % (seed, n), boxes, scores, t,
                    class_ids=class_ids, batch_offsets=offsets,
                    meta={"seed": seed})
