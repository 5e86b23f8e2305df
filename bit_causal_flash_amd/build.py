"""Build the HIP library (libflamia.so) in-tree for gfx950 with hipcc.

    python -m bit_causal_flash_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled, then
linked into one shared library next to this file."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libflamia.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quant.hip", "worklist.hip", "fwd.hip", "bwd.hip", "api.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I" + INCLUDE, "-I" + CSRC,
         "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    objdir = tempfile.mkdtemp(prefix="flamia_build_")
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                        if "not a recognized feature" not in line)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % (res.stdout + res.stderr))
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    os.rmdir(objdir)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
