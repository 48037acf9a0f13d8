"""Build the gfx950 HIP library ``libgla_mi355x.so`` in-tree.

Usage: ``python -m gated_deltanet_gla_amd.build`` (or ``build()``).  Every
HIP source under ``csrc/`` is compiled with hipcc for gfx950 and linked into
one shared library next to this file.  Compiles run in parallel; the result
replaces the previous library atomically.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgla_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # keep the compiler from forming packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-fvisibility=hidden",
]


def sources():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    return srcs


def _compile(src, obj, extra):
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None, jobs: int | None = None) -> str:
    """Compile every source and link the library; returns its path."""
    extra = list(extra_flags or [])
    srcs = sources()
    tmp = tempfile.mkdtemp(prefix="gla_build_")
    try:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        jobs = jobs or min(8, len(srcs))
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            futs = {ex.submit(_compile, s, o, extra): s for s, o in zip(srcs, objs)}
            for f in cf.as_completed(futs):
                out = f.result()
                if verbose and out.strip():
                    print(out)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}")
        shutil.copyfile(tmp_lib, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
