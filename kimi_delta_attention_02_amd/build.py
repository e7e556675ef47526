"""Compile the HIP library (gfx950) in-tree: kimi_delta_attention_02_amd/libkda.so.

Each source is compiled to an object of its own, in parallel, and the objects
are linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkda.so")
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

# packed fp32 instructions are kept out of the device code on purpose
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))) + [
        os.path.join(PKG, "csrc", "kda_api.cpp")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source into libkda.so (always rebuilds); returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    tmpdir = tempfile.mkdtemp(prefix="kda_build_")
    try:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([hipcc] + HIPCC_FLAGS + inc + ["-c", src, "-o", obj])
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
