"""Loader for the hand-built fixtures under tests/golden/ (each file carries
its citation and the arithmetic behind its expected values)."""
import glob
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_cases():
    """Yield (name, boxes, scores, t, class_ids, batch_offsets, expected_keep)."""
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        name = os.path.splitext(os.path.basename(path))[0]
        with open(path) as f:
            d = json.load(f)
        assert d.get("citation"), name
        boxes = np.asarray(d["boxes"], dtype=np.float32).reshape(-1, 4)
        scores = np.asarray(d["scores"], dtype=np.float32)
        cls = None if "class_ids" not in d else np.asarray(d["class_ids"], dtype=np.int32)
        offs = None if "batch_offsets" not in d else np.asarray(d["batch_offsets"], dtype=np.int64)
        cases = d.get("cases") or [{"iou_threshold": d["iou_threshold"],
                                    "expected_keep": d["expected_keep"]}]
        for k, c in enumerate(cases):
            label = name if len(cases) == 1 else "%s[%d]" % (name, k)
            out.append((label, boxes, scores, float(c["iou_threshold"]), cls, offs,
                        np.asarray(c["expected_keep"], dtype=np.int64)))
    return out


def load_raw(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        return json.load(f)
