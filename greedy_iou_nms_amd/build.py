"""Build libgreedy_nms.so for gfx950 with hipcc (in-tree, next to this file).

Flags that matter for correctness:
  -ffp-contract=off   the IoU expression must round every step separately,
                      exactly as the float32 definition does (no FMA fusion);
  -fhip-fp32-correctly-rounded-divide-sqrt
                      the literal-division path must round correctly;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keeps the compiler from emitting packed fp32 ops.

Every build also checks the compiler's resource report for the kernels whose
waves hand work to each other through LDS flags (the sweeps): no scratch
memory, no spilled VGPRs, and fewer than 256 VGPRs.  A build that breaks one
of these limits fails instead of producing a library.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libgreedy_nms.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["radix.hip", "team_sort.hip", "mask.hip", "sweep.hip", "matrix.hip", "nms_api.cpp"]

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE,
]

# Kernels whose resource report is checked, by a substring of their mangled
# name.  The plain sweep kernel of a build that held 2048 list entries per
# register set compiled to exactly 256 VGPRs and returned wrong kept sets.
# The team sort's workgroups wait on one another, so all of them must be
# resident at once; scratch memory could limit that.
GUARDED_KERNELS = ("12sweep_kernel", "17mask_sweep_kernel", "18group_sweep_kernel",
                   "16small_nms_kernel", "16team_sort_kernel", "18team_sample_kernel")
MAX_VGPRS = 255


def parse_resource_usage(text: str) -> dict:
    """Per kernel (mangled name): the fields of clang's
    -Rpass-analysis=kernel-resource-usage remarks, as integers."""
    usage = {}
    current = None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            current = usage.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(-?\d+)\s", line + " ")
        if m and current is not None:
            current[m.group(1).strip()] = int(m.group(2))
    return usage


def check_resources(usage: dict) -> list:
    """Violations of the guarded kernels' limits, as messages."""
    bad = []
    for name, u in usage.items():
        if not any(g in name for g in GUARDED_KERNELS):
            continue
        if u.get("VGPRs", 0) > MAX_VGPRS:
            bad.append("%s: %d VGPRs (limit %d)" % (name, u["VGPRs"], MAX_VGPRS))
        if u.get("ScratchSize [bytes/lane]", 0) != 0:
            bad.append("%s: %d bytes of scratch per lane" % (name, u["ScratchSize [bytes/lane]"]))
        if u.get("VGPRs Spill", 0) != 0:
            bad.append("%s: %d VGPRs spilled" % (name, u["VGPRs Spill"]))
    return bad


def build(verbose: bool = False, extra=()) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *extra, "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
    failed = []
    usage = {}
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        usage.update(parse_resource_usage(text))
        # the host pass does not know the packed-fp32 feature flag; that
        # notice, and the resource remarks, are dropped
        shown = []
        skip_source_echo = False
        for line in text.splitlines(True):
            if "packed-fp32-ops" in line:
                continue
            if "kernel-resource-usage" in line:
                skip_source_echo = True
                continue
            if skip_source_echo and (line.lstrip().startswith("|") or
                                     re.match(r"\s*\d+ \|", line)):
                continue
            skip_source_echo = False
            shown.append(line)
        if "".join(shown).strip():
            sys.stderr.write("".join(shown))
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    bad = check_resources(usage)
    if bad:
        raise RuntimeError("kernel resource limits broken:\n  " + "\n  ".join(bad))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
