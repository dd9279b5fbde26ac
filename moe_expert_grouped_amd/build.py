"""Build the HIP library libmoe_gfx950.so in-tree with hipcc (gfx950 only).

    python -m moe_expert_grouped_amd.build        # or build() from Python

Every .hip file under csrc/ is compiled to an object in parallel, then linked
into one shared library next to this file.  gg_inst.hip is compiled once per
(epilogue, B layout, dtype, B cache policy) combination of the grouped GEMM
(GG_VARIANTS), so
the heavy template instantiations build side by side.  The build always
recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_gfx950.so")
PEAK_SRC = os.path.join(HERE, "peak", "peak.hip")
PEAK_LIB = os.path.join(HERE, "libmoe_peak_gfx950.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


# (epilogue, B stored [K][N], fp16) of every grouped GEMM instantiation the
# dispatcher in grouped_gemm.hip declares: store and SiLU*up in both layouts
# and dtypes, the weighted scatter for [K][N] weights.
# (epilogue, [K][N] B, fp16, non-temporal B): the non-temporal weight loads
# exist for the [K][N] layouts only
# (.., 1): the fused gate/up form (the permutation inside the kernel), bf16
# [K][N] weights, both cache policies
GG_VARIANTS = [(e, kn, f, 0, 0) for e in (0, 1) for kn in (1, 0) for f in (0, 1)] + \
              [(2, 1, 0, 0, 0), (2, 1, 1, 0, 0)] + \
              [(e, 1, f, 1, 0) for e in (0, 1, 2) for f in (0, 1)] + \
              [(1, 1, 0, nt, 1) for nt in (0, 1)]


def _compile(job) -> str:
    src, defs = job
    tag = "".join("_%s%d" % (k[3:].lower(), v) for k, v in defs)
    obj = os.path.join(OBJ, os.path.basename(src) + tag + ".o")
    if src == PEAK_SRC:
        obj = os.path.join(OBJ, "peak_" + os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *["-D%s=%d" % kv for kv in defs], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        if os.path.basename(src) == "gg_inst.hip":
            jobs += [(src, (("GG_EPI", e), ("GG_KN", kn), ("GG_FP16", f), ("GG_NT", nt), ("GG_LP", lp)))
                     for e, kn, f, nt, lp in GG_VARIANTS]
        else:
            jobs.append((src, ()))
    # the instantiations are the slow ones: start them first
    jobs.sort(key=lambda j: not j[1])
    jobs.append((PEAK_SRC, ()))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    peak_obj = objs.pop()
    for lib, lib_objs in ((LIB, objs), (PEAK_LIB, [peak_obj])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *lib_objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
