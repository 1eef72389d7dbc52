"""Helpers for GPU tests: move numpy workloads to the device and run the HIP
library through its Python binding (which calls the C ABI)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_nms(boxes, scores, t, class_ids=None, batch_offsets=None, workspace=None):
    import greedy_iou_nms_amd as g
    dev = device()
    keep = g.nms(to_dev(np.asarray(boxes, np.float32).reshape(-1, 4), dev),
                 to_dev(np.asarray(scores, np.float32), dev), t,
                 to_dev(class_ids, dev), to_dev(batch_offsets, dev), workspace=workspace)
    return keep.cpu().numpy()


def note(msg):
    """Print a line naming the case before GPU work (survives a lost box)."""
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()
