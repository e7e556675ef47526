"""Compile the HIP library (gfx950) in-tree: kimi_delta_attention_02_amd/libkda.so."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkda.so")
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

# packed fp32 instructions are kept out of the device code on purpose
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))) + [
        os.path.join(PKG, "csrc", "kda_api.cpp")]


def build(verbose: bool = False) -> str:
    """Compile every source into libkda.so (always rebuilds); returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"),
                                   "-I", os.path.join(PKG, "csrc")] + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
