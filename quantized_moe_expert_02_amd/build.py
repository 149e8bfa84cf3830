"""Build the HIP library (libmoe_w4a16.so) in-tree for gfx950 with hipcc.

Each source is compiled to its own object (in parallel, under _build/), then
the objects are linked into the shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_w4a16.so")
OBJ_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 instructions stay off: hipcc emits them on its own
         # from plain float code, and the library does not rely on them.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def compile_command(src: str, obj: str):
    return ["hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            "-c", src, "-o", obj]


def link_command(objs, out: str):
    return ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return r.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [compile_command(s, o) for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, out), c in zip(results, cmds):
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(c) + "\n" + out)
        if verbose and out:
            print(out)
    tmp = LIB + ".tmp"
    rc, out = _run(link_command(objs, tmp))
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
