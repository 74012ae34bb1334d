"""Build libssm_mi355x.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU ops
disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssm_mi355x.so")
# measurement-only microbenchmarks (include/ssm_microbench.h), a library of their own
MB_LIB = os.path.join(HERE, "libssm_microbench.so")
MB_SOURCE = ("microbench.hip", [])
SOURCES = [("api.cpp", []), ("scan_host.hip", []), ("ssd_kernels.hip", []), ("step_kernels.hip", []), ("conv_kernels.hip", []), ("scan_bwd.hip", [])] + [
    ("scan_inst.hip", ["-DSSM_R=%d" % rr, "-DSSM_XB=%d" % xb, "-DSSM_DB=%d" % db, "-DSSM_S=%d" % sv])
    for rr, sv in ((4, 32), (8, 32), (4, 16), (4, 8), (4, 4), (4, 2), (4, 1), (8, 2), (16, 1))
    for xb in (1, 0) for db in (1, 0)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast"]


def _compile(item) -> str:
    src, defs = item
    tag = "_".join(d.split("=")[-1] for d in defs)
    out = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + defs + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for %s" % src)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES) + 1, os.cpu_count() or 8, 16)) as ex:
        objs = list(ex.map(_compile, SOURCES + [MB_SOURCE]))
    mb_obj = objs.pop()
    for lib, parts in ((LIB, objs), (MB_LIB, [mb_obj])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + parts
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("link failed")
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
