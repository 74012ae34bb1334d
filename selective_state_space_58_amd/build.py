"""Build libssm_mi355x.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU ops
disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssm_mi355x.so")
# measurement-only microbenchmarks (include/ssm_microbench.h), a library of their own
MB_LIB = os.path.join(HERE, "libssm_microbench.so")
MB_SOURCE = ("microbench.hip", [])
SOURCES = [("api.cpp", []), ("scan_host.hip", []), ("ssd_kernels.hip", []), ("step_kernels.hip", []), ("conv_kernels.hip", []), ("scan_bwd.hip", []), ("scan_long.hip", []), ("ssd_rec.hip", [])] + [
    ("scan_inst.hip", ["-DSSM_R=%d" % rr, "-DSSM_XB=%d" % xb, "-DSSM_DB=%d" % db, "-DSSM_S=%d" % sv])
    for rr, sv in ((4, 32), (8, 32), (4, 16), (4, 8), (4, 4), (4, 2), (4, 1), (8, 2), (16, 1))
    for xb in (1, 0) for db in (1, 0)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast"]


def source_digest(csrc: str = CSRC, include: str = INCLUDE) -> str:
    """SHA-256 (hex) over the library's sources: every file of csrc/ and every header of include/,
    by name and content, in sorted order.  The build embeds it in the library so that a loader can
    tell a build made from other sources."""
    h = hashlib.sha256()
    files = [("csrc/" + f, os.path.join(csrc, f)) for f in sorted(os.listdir(csrc))
             if os.path.isfile(os.path.join(csrc, f))]
    files += [("include/" + f, os.path.join(include, f)) for f in sorted(os.listdir(include)) if f.endswith(".h")]
    for name, path in files:
        with open(path, "rb") as fh:
            data = fh.read()
        h.update(name.encode() + b"\0" + str(len(data)).encode() + b"\0" + data)
    return h.hexdigest()


# marker in front of the embedded digest (api.cpp stores "<marker><64 hex digits>")
DIGEST_MARKER = b"ssm-source-sha256:"


def built_digest(lib: str = LIB) -> str | None:
    """The source digest embedded in a built library file (read from its bytes, without loading it);
    None when the file is missing or carries no digest."""
    try:
        with open(lib, "rb") as fh:
            data = fh.read()
    except OSError:
        return None
    i = data.find(DIGEST_MARKER)
    if i < 0:
        return None
    d = data[i + len(DIGEST_MARKER):i + len(DIGEST_MARKER) + 64]
    try:
        d = d.decode("ascii")
    except UnicodeDecodeError:
        return None
    return d if len(d) == 64 and all(ch in "0123456789abcdef" for ch in d) else None


def stale_reason(lib: str = LIB, csrc: str = CSRC, include: str = INCLUDE) -> str | None:
    """None when `lib` exists and was built from the sources in csrc/ and include/, else why not."""
    if not os.path.exists(lib):
        return "%s is not built" % lib
    b = built_digest(lib)
    if b is None:
        return "%s carries no source digest" % lib
    s = source_digest(csrc, include)
    if b != s:
        return "%s was built from other sources (built %s, sources %s)" % (lib, b[:16], s[:16])
    return None


def _compile(item) -> str:
    src, defs = item
    tag = "_".join(d.split("=")[-1] for d in defs if not d.startswith("-DSSM_SOURCE_DIGEST"))
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
    digest = source_digest()
    items = [(src, defs + ['-DSSM_SOURCE_DIGEST="%s"' % digest] if src == "api.cpp" else defs)
             for src, defs in SOURCES]
    with ThreadPoolExecutor(min(len(SOURCES) + 1, os.cpu_count() or 8, 16)) as ex:
        objs = list(ex.map(_compile, items + [MB_SOURCE]))
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
