"""Benchmark: greedy IoU NMS on one MI355X.

One step = one full NMS call (sort, IoU mask, sweep, compaction and the
kept-count read-back) over the N = 65536 single-image workload (half uniform
boxes, half clustered; threshold 0.5), inputs already resident in device
memory.  Prints one JSON line:

  value          boxes/s over the timed steps (whole job, one GPU)
  roofline       the dominant kernel of the timed steps (at this size the
                 fused IoU-mask launch, whose sweep workgroup runs beside the
                 mask) against the published fp32 vector peak (157.3 TFLOP/s),
                 counting 13 algorithmic fp32 operations per box pair for every
                 pair of the triangle, timed with HIP events on the launch
                 stream
  mask_kernel_alone, sweep_alone
                 the mask and the sweep as separate launches (a few extra
                 steps), so each is measured on its own line
  e2e_roofline   max(VALU time of all pairs, HBM time of the mask's algorithmic
                 bytes) over the measured median call time
  cpu_baseline   the CPU oracle on the same workload, on this host
  n8192          the same measurement on the N = 8192 clustered workload
  matrix_nms     Matrix NMS (Gaussian decay, score threshold 0.1, sigma 0.5)
                 on the boxes and scores of both workloads: call time, stage
                 times, pair evaluations per second of its two pairwise
                 kernels and their dense-equivalent fraction of the fp32
                 vector peak; parity with the CPU oracle at N = 8192
  near_threshold_pairs
                 pairs the oracle evaluated with |IoU - t| <= 1e-6, per
                 workload (from the oracle run of the cpu_baseline leg)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --copy-calibration BYTES
         (device-to-device copies of a known size, run under rocprofv3 --pmc
          to scale the FETCH_SIZE / WRITE_SIZE counters to bytes)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# fp32 ops per box pair counted as the algorithmic work of the IoU test:
# 4 max/min, 2 sub, 2 clamps, 1 mul, 1 add, 1 sub, 1 div, 1 compare
OPS_PER_PAIR = 13
# MI355X's published fp32 vector peak (dense), TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3
# The rate at which plain fp32 add / sub / mul and bitwise ops issue (one
# wave64 instruction per 2 cycles per SIMD: 256 x 4 x 32 x 2.4 GHz), quoted
# beside the published peak as a side figure only.
FP32_ISSUE_RATE_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
COUNTED = ("algorithmic fp32 operations of the IoU test, 13 per box pair, over every pair "
           "of the triangle (pairs the overlap pre-test rejects count as done)")
HBM_PEAK_GBS = 8000.0
# column tiles per mask work item for one image: a row's words are written
# from the start of the strip holding its own tile
MASK_STRIP = 8


def _measure(w, steps, warmup, fuse=True):
    """Time `steps` calls after `warmup` untimed ones, as a user calls the
    library (``nms``: every call returns once its result is complete, so the
    host clock around a call is its end-to-end time), then `steps` calls of
    ``nms_profiled`` (HIP events on the launch stream around every stage) for
    the stage times.  fuse=False: the mask and the sweep as separate
    launches; every timed call is then a profiled one."""
    import numpy as np
    import torch

    import greedy_iou_nms_amd as g

    dev = torch.device("cuda:0")
    boxes = torch.from_numpy(w.boxes).to(dev)
    scores = torch.from_numpy(w.scores).to(dev)
    cls = None if w.class_ids is None else torch.from_numpy(w.class_ids).to(dev)
    offs = None if w.batch_offsets is None else torch.from_numpy(w.batch_offsets).to(dev)
    ws = g.Workspace(dev)
    out = torch.empty(w.n, dtype=torch.int64, device=dev)

    def profiled():
        return g.nms_profiled(boxes, scores, w.iou_threshold, cls, offs, workspace=ws, out=out,
                              fuse=fuse)

    def call():
        if not fuse:
            return profiled()[0]
        return g.nms(boxes, scores, w.iou_threshold, cls, offs, workspace=ws, out=out)

    first = None
    for _ in range(warmup):
        keep = call()
        if first is None:
            first = keep.cpu().numpy().copy()
        profiled()
    torch.cuda.synchronize()
    call_ms = []
    t0 = time.perf_counter()
    for _ in range(steps):
        t1 = time.perf_counter()
        keep = call()
        call_ms.append(1000.0 * (time.perf_counter() - t1))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    last = keep.cpu().numpy().copy()
    stage_sum = {s: 0.0 for s in g.STAGES}
    for _ in range(steps):
        _, st = profiled()
        for k, v in st.items():
            stage_sum[k] += v
    torch.cuda.synchronize()
    deterministic = first is None or bool(np.array_equal(first, last))
    return {
        "elapsed": elapsed,
        "stage_ms": {k: v / steps for k, v in stage_sum.items()},
        "call_ms": {"median": float(np.median(call_ms)), "min": float(np.min(call_ms))},
        "keep": last,
        "deterministic": deterministic,
    }


# Counter-derived HBM traffic of the dominant kernel (the fused mask + sweep
# launch), recorded in a profile summary together with a hash of the
# kernel's sources; reported only while the sources are unchanged.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_mask_sweep_kernel_n65536_large_mixed.md")
MASK_SOURCES = [os.path.join(ROOT, "greedy_iou_nms_amd", "csrc", f)
                for f in ("mask_core.h", "sweep.hip", "nms_internal.h")]


def mask_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in MASK_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic():
    """(bytes per launch, detail) from the recorded counters, or (None, reason)."""
    if not os.path.exists(TRAFFIC_RECORD):
        return None, "no counter record"
    rec = None
    with open(TRAFFIC_RECORD) as fh:
        for line in fh:
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
    if rec is None:
        return None, "no counter record"
    if rec.get("source_sha256") != mask_source_sha256():
        return None, "mask kernel changed since the counters were taken"
    detail = {k: rec[k] for k in ("kernel", "fetch_bytes", "write_bytes", "fetch_scale",
                                  "write_scale", "record") if k in rec}
    return rec["fetch_bytes"] + rec["write_bytes"], detail


def _dense_band_bytes(w):
    """Bytes of a mask kernel that writes every word of the row band (the
    dense form, which this library writes only when a tile's list of nonzero
    words overflows), plus the sorted boxes and areas read once."""
    n = w.n
    words = (n + 63) // 64
    strip = MASK_STRIP
    total = 0
    for r in range(words):
        rows = min(64, n - 64 * r)
        total += rows * (words - (r // strip) * strip) * 8
    return total + 20 * n


def _mask_nonzero_words(w):
    """Nonzero 64-bit words of the suppression mask of one single-image
    call, counted on the device from the library's dense export (outside any
    timed region)."""
    import torch
    import greedy_iou_nms_amd as g
    dev = torch.device("cuda:0")
    m, _ = g.debug_mask(torch.from_numpy(w.boxes).to(dev), torch.from_numpy(w.scores).to(dev),
                        w.iou_threshold)
    nnz = int(torch.count_nonzero(m).item())
    del m
    torch.cuda.empty_cache()
    return nnz


def _mask_sparse_bytes(w, nnz):
    """Bytes the mask must move for one single-image call when it writes
    only the nonzero words: the sorted boxes and areas read once (20 B per
    box) and every nonzero word written once with its column (12 B)."""
    return 20 * w.n + 12 * nnz


def _sweep_dense_bytes(w, keep):
    """Bytes a dense-row sweep reads: the 64 diagonal words of every row tile
    and, for every kept box at sorted position p, its words right of its own
    tile (W - p // 64 - 1 of them).  This sweep reads sparse lists instead,
    so this is the dense equivalent the rate is quoted against."""
    import numpy as np
    n = w.n
    words = (n + 63) // 64
    order = np.lexsort((np.arange(n), -w.scores.astype(np.float64)))
    pos = np.empty(n, np.int64)
    pos[order] = np.arange(n)
    kept_pos = pos[np.asarray(keep, np.int64)]
    return int(8 * n + 8 * np.sum(words - kept_pos // 64 - 1))


def _copy_calibration(nbytes, launches=5):
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": launches}), flush=True)


def _pairs(w):
    import numpy as np
    if w.batch_offsets is None and w.class_ids is None:
        return w.n * (w.n - 1) // 2
    img = np.repeat(np.arange(len(w.batch_offsets) - 1), np.diff(w.batch_offsets))
    key = img * 100000 + w.class_ids.astype(np.int64)
    _, counts = np.unique(key, return_counts=True)
    return int(np.sum(counts * (counts - 1) // 2))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Algorithmic fp32 ops per (father, child) pair of the two pairwise Matrix
# NMS kernels: the IoU (4 max/min, 2 sub, 2 clamps, mul, add, sub, div) and
# the running maximum (overlap), or the IoU, its square, the difference with
# the father's maximum, the scaling by sigma and the compare (decay).
MATRIX_OVERLAP_INSTR = 13
MATRIX_DECAY_INSTR = 16
MATRIX_T, MATRIX_SIGMA = 0.1, 0.5


def _measure_matrix(w, steps, warmup):
    import numpy as np
    import torch

    import greedy_iou_nms_amd as g

    dev = torch.device("cuda:0")
    boxes = torch.from_numpy(w.boxes).to(dev)
    scores = torch.from_numpy(w.scores).to(dev)
    ws = g.Workspace(dev)
    out = torch.empty(w.n, dtype=torch.int64, device=dev)
    for _ in range(warmup):
        g.matrix_nms(boxes, scores, MATRIX_T, MATRIX_SIGMA, workspace=ws, out=out)
    torch.cuda.synchronize()
    call_ms, stages = [], []
    for _ in range(steps):
        t1 = time.perf_counter()
        keep = g.matrix_nms(boxes, scores, MATRIX_T, MATRIX_SIGMA, workspace=ws, out=out)
        call_ms.append(1000.0 * (time.perf_counter() - t1))
    for _ in range(max(3, steps // 2)):
        _, st = g.matrix_nms_profiled(boxes, scores, MATRIX_T, MATRIX_SIGMA, workspace=ws,
                                      out=out)
        stages.append(st)
    keep = keep.cpu().numpy().copy()
    pairs = w.n * (w.n - 1) // 2
    med = float(np.median(call_ms))
    st = {k: float(np.median([x[k] for x in stages])) for k in stages[0]}
    res = {"workload": w.name, "n": w.n, "score_threshold": MATRIX_T, "sigma": MATRIX_SIGMA,
           "ms_per_call": {"median": med, "min": float(np.min(call_ms))},
           "boxes_per_s": w.n / (med * 1e-3), "stage_ms": st, "kept": int(keep.size)}
    for name, key, instr in (("overlap_max", "overlap_max", MATRIX_OVERLAP_INSTR),
                             ("decay", "decay", MATRIX_DECAY_INSTR)):
        rate = pairs / (st[key] * 1e-3)
        res[name + "_pairs_per_s"] = rate
        # dense-equivalent: every pair counted, also those the kernel skips
        # because they cannot overlap, so this is not executed utilisation
        res[name + "_dense_equivalent_frac_of_157tf"] = (
            instr * rate / (FP32_VECTOR_PEAK_TFLOPS * 1e12))
    return res, keep


def _workload_line(w, r):
    """Per-workload figures shared by the main line and the n8192 object."""
    pairs = _pairs(w)
    ms = r["call_ms"]["median"]
    return {
        "workload": w.name,
        "boxes_per_s": w.n / (ms * 1e-3),
        "pairwise_iou_per_s": pairs / (ms * 1e-3),
        "pairwise_iou_per_s_mask_stage": pairs / (r["stage_ms"]["mask"] * 1e-3),
        "ms_per_call": r["call_ms"],
        "stage_ms": r["stage_ms"],
        "kept": int(r["keep"].size),
        "deterministic": r["deterministic"],
    }


def _table(steps, warmup):
    """Per workload: the library's call time and stage times, pair rates,
    exact parity with the oracle, 10 identical results in a row, and the
    oracle's own time (single-threaded)."""
    import numpy as np
    import torch

    import greedy_iou_nms_amd as g
    import oracle
    import workloads

    dev = torch.device("cuda:0")
    for idx in (1, 2, 3, 4, 5):
        w = workloads.config(idx, seed=0)
        r = _measure(w, steps, warmup)
        pairs = _pairs(w)
        ms = r["call_ms"]["median"]
        mask_ms = r["stage_ms"]["mask"]
        b = torch.from_numpy(w.boxes).to(dev)
        sc = torch.from_numpy(w.scores).to(dev)
        cl = None if w.class_ids is None else torch.from_numpy(w.class_ids).to(dev)
        of = None if w.batch_offsets is None else torch.from_numpy(w.batch_offsets).to(dev)
        runs = [g.nms(b, sc, w.iou_threshold, cl, of).cpu().numpy() for _ in range(10)]
        t0 = time.perf_counter()
        want, border = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, w.class_ids,
                                    w.batch_offsets, return_borderline=True)
        cpu_s = time.perf_counter() - t0
        single = w.class_ids is None and w.batch_offsets is None
        line = {
            "config": idx, "workload": w.name, "n": w.n, "kept": int(r["keep"].size),
            "ms_per_call": r["call_ms"], "boxes_per_s": w.n / (ms * 1e-3),
            "stage_ms": r["stage_ms"], "pairs": pairs,
            "iou_per_s_mask_stage": pairs / (mask_ms * 1e-3),
            "iou_per_s_call": pairs / (ms * 1e-3),
            "mask_stage_frac_of_157tf": OPS_PER_PAIR * pairs / (mask_ms * 1e-3) /
                                        (FP32_VECTOR_PEAK_TFLOPS * 1e12),
            "mask_dense_equivalent_gbs": (_dense_band_bytes(w) / (mask_ms * 1e-3) / 1e9
                                          if single else None),
            "parity_vs_oracle": bool(np.array_equal(r["keep"], want)),
            "ten_runs_identical": all(np.array_equal(x, runs[0]) for x in runs),
            "oracle_s_one_thread": cpu_s, "near_threshold_pairs": int(border),
        }
        print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the N=65536 workload as the library runs it (for profiler runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run device copies of BYTES bytes (counter calibration)")
    ap.add_argument("--trace-config", type=int, default=0, metavar="K",
                    help="only time workload K (1..5) as the library runs it (for profiler runs)")
    ap.add_argument("--table", action="store_true",
                    help="one JSON line per workload 1..5: call time, stage times, pair rates, "
                         "parity with the oracle, 10-run determinism, oracle time")
    ap.add_argument("--separate", action="store_true",
                    help="with --main-only: the mask and the sweep as separate launches "
                         "(for profiler runs of the mask kernel alone)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs the whole path on "
              "a single MI355X (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        _copy_calibration(args.copy_calibration)
        return

    import workloads

    if args.table:
        _table(args.steps, args.warmup)
        return

    if args.trace_config:
        wt = workloads.config(args.trace_config, seed=0)
        rt = _measure(wt, args.steps, args.warmup)
        print(json.dumps({"workload": wt.name, "n": wt.n, "steps": args.steps,
                          "ms_per_call": rt["call_ms"], "stage_ms": rt["stage_ms"]}))
        return

    w = workloads.config(5, seed=0)
    if args.separate:
        rs = _measure(w, args.steps, args.warmup, fuse=False)
        print(json.dumps({"workload": w.name, "n": w.n, "steps": args.steps,
                          "separate_launches": True, "ms_per_call": rs["call_ms"],
                          "stage_ms": rs["stage_ms"]}))
        return
    r = _measure(w, args.steps, args.warmup)
    ms_per_step = 1000.0 * r["elapsed"] / args.steps
    pairs = _pairs(w)
    launch_ms = r["stage_ms"]["mask"]
    achieved = OPS_PER_PAIR * pairs / (launch_ms * 1e-3) / 1e12
    traffic, traffic_detail = _traffic()
    dense_bytes = _dense_band_bytes(w)
    # the nonzero words come from an extra export call: not in the profiled
    # main-only runs, whose traces hold the timed kernels only
    nnz = None if args.main_only else _mask_nonzero_words(w)
    alg_bytes = None if nnz is None else _mask_sparse_bytes(w, nnz)

    line = {
        "metric": "NMS boxes/s and pairwise IoU/s at N=8192 and N=65536 (1 MI355X); % of roofline",
        "value": w.n / (ms_per_step * 1e-3),
        "unit": "boxes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "iou_threshold": w.iou_threshold,
                   "seed": 0, "input_sha256": w.sha256()[:16]},
    }
    line.update({k: v for k, v in _workload_line(w, r).items() if k != "workload"})
    line["roofline"] = {
        "kernel": "mask_sweep_kernel (IoU suppression bitmask; the sweep's workgroup runs "
                  "beside it)",
        "bound": "alu",
        "achieved": achieved,
        "peak": FP32_VECTOR_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "counted": COUNTED,
        "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
        "traffic": traffic,
        "traffic_detail": traffic_detail,
        "algorithmic_bytes": alg_bytes,
        "algorithmic_bytes_counted": "20 B per box read (sorted box, area) + 12 B per nonzero "
                                     "mask word written (value, column)",
        "nonzero_mask_words": nnz,
        "dense_band_bytes": dense_bytes,
        "ops_per_pair": OPS_PER_PAIR,
        "pairs_per_launch": pairs,
        "launch_ms": launch_ms,
        "side_frac_of_fp32_issue_rate_78tops": achieved / FP32_ISSUE_RATE_TOPS,
        "executed_valu": "profiles/valu_mask_kernels_n65536_large_mixed.md",
    }

    if not args.main_only:
        # the mask and the sweep as separate launches, each on its own line
        sep_steps = max(1, min(args.steps, 20))
        s = _measure(w, sep_steps, min(args.warmup, 3), fuse=False)
        m_ms = s["stage_ms"]["mask"]
        m_ach = OPS_PER_PAIR * pairs / (m_ms * 1e-3) / 1e12
        line["mask_kernel_alone"] = {
            "kernel": "mask_kernel (separate launch)", "launch_ms": m_ms, "achieved": m_ach,
            "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s", "counted": COUNTED,
            "frac": m_ach / FP32_VECTOR_PEAK_TFLOPS, "steps": sep_steps,
        }
        sw_ms = s["stage_ms"]["sweep"]
        dense = _sweep_dense_bytes(w, s["keep"])
        line["sweep_alone"] = {
            "kernel": "sweep_kernel (separate launch, one workgroup)", "ms": sw_ms,
            "dense_equivalent_bytes": dense, "dense_equivalent_gbs": dense / (sw_ms * 1e-3) / 1e9,
            "us_per_row_tile": 1000.0 * sw_ms / ((w.n + 63) // 64), "steps": sep_steps,
        }
        valu_ms = 1000.0 * OPS_PER_PAIR * pairs / (FP32_VECTOR_PEAK_TFLOPS * 1e12)
        hbm_ms = 1000.0 * (alg_bytes or 0) / (HBM_PEAK_GBS * 1e9)
        roof_ms = max(valu_ms, hbm_ms)
        line["e2e_roofline"] = {
            "roofline_ms": roof_ms, "valu_ms": valu_ms, "hbm_ms": hbm_ms,
            "measured_ms": r["call_ms"]["median"],
            "ratio": roof_ms / r["call_ms"]["median"],
        }

        w2 = workloads.config(2, seed=0)
        r2 = _measure(w2, args.steps, args.warmup)
        line["n8192"] = _workload_line(w2, r2)

        msteps = max(3, min(args.steps, 20))
        m2, k2 = _measure_matrix(w2, msteps, min(args.warmup, 3))
        m5, _ = _measure_matrix(w, msteps, min(args.warmup, 3))
        line["matrix_nms"] = {"n8192": m2, "n65536": m5}
        if not args.no_cpu:
            import numpy as np

            import oracle
            line["matrix_nms"]["n8192"]["parity_vs_oracle"] = bool(np.array_equal(
                k2, oracle.c_matrix_nms(w2.boxes, w2.scores, MATRIX_T, MATRIX_SIGMA)))

    if not args.no_cpu:
        import numpy as np

        import oracle
        t0 = time.perf_counter()
        want, border5 = oracle.c_nms(w.boxes, w.scores, w.iou_threshold, return_borderline=True)
        cpu_s = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": w.n / cpu_s, "unit": "boxes/s", "cores": 1, "kind": "oracle",
            "sample": "the full %s workload, one single-threaded run (%.1f s) on %s; host has %d "
                      "usable cores" % (w.name, cpu_s, _cpu_model(),
                                        len(os.sched_getaffinity(0))),
        }
        line["parity_vs_oracle"] = bool(np.array_equal(r["keep"], want))
        near = {w.name: border5}
        if "n8192" in line:
            want2, border2 = oracle.c_nms(w2.boxes, w2.scores, w2.iou_threshold,
                                          return_borderline=True)
            near[w2.name] = border2
            line["n8192"]["parity_vs_oracle"] = bool(np.array_equal(r2["keep"], want2))
        line["near_threshold_pairs"] = near
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
