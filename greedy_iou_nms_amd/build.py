"""Build libgreedy_nms.so for gfx950 with hipcc (in-tree, next to this file).

Flags that matter for correctness:
  -ffp-contract=off   the IoU expression must round every step separately,
                      exactly as the float32 definition does (no FMA fusion);
  -fhip-fp32-correctly-rounded-divide-sqrt
                      the literal-division path must round correctly;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keeps the compiler from emitting packed fp32 ops.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libgreedy_nms.so")
# instruction issue-rate probe for the roofline figures (bench.py --valu-rates)
PROBE = os.path.join(HERE, "valu_rate_probe")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["radix.hip", "mask.hip", "sweep.hip", "matrix.hip", "nms_api.cpp"]

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE,
]


def build(verbose: bool = False, extra=()) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
    failed = []
    probe_cmd = [HIPCC, "--offload-arch=" + ARCH, "-O2", "-Wno-unused-result",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 os.path.join(CSRC, "valu_rate_probe.hip"), "-o", PROBE + ".tmp"]
    procs.append(("valu_rate_probe.hip", subprocess.Popen(probe_cmd, stdout=subprocess.PIPE,
                                                          stderr=subprocess.STDOUT)))
    for src, p in procs:
        out, _ = p.communicate()
        # the host pass does not know the packed-fp32 feature flag; that
        # notice is expected and dropped
        text = "".join(line for line in out.decode(errors="replace").splitlines(True)
                       if "packed-fp32-ops" not in line)
        if text.strip():
            sys.stderr.write(text)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    os.replace(PROBE + ".tmp", PROBE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
