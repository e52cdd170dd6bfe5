"""Build libckks_mi355x.so (HIP, gfx950) in place with hipcc.

Each source is compiled to an object of its own in parallel (a temporary
directory), then the objects are linked into the shared library."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libckks_mi355x.so")
SOURCES = ["ctx.hip", "ntt.hip", "kernels.hip", "keyswitch.hip", "rescale.hip", "ops.hip", "noalloc.hip", "probe.hip"]
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmpdir = tempfile.mkdtemp(prefix="ckks_build_")
    try:
        objs = [os.path.join(tmpdir, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[hipcc] + FLAGS + ["-c", "-o", o, os.path.join(SRC, s)] for s, o in zip(SOURCES, objs)]
        jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
