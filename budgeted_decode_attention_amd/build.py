"""Builds libkvevict.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m budgeted_decode_attention_amd.build [-v]
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvevict.so")
ARCH = os.environ.get("KVEVICT_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compiles every source to an object in parallel, then links the shared
    library atomically (write to a temp name, then rename)."""
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objdir = tempfile.mkdtemp(prefix="kvevict_obj_")
    try:
        procs, objs = [], []
        srcs = sources()
        for s in srcs:
            o = os.path.join(objdir, os.path.basename(s) + ".o")
            objs.append(o)
            cmd = [cc, *FLAGS, *inc, "-c", s, "-o", o]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        for p in procs:
            _wait(p, verbose)
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{text}")
    if verbose and text.strip():
        print(text, flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
