"""Build libattnres.so (gfx950) in-tree with hipcc.

    python -m transformer_depth_wise_amd.build [--incremental]

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libattnres.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "phase1.hip", "merge.hip", "full.hip", "backward.hip", "backward_p2.hip",
           "backward_p1_bf16.hip", "backward_p1_f32.hip", "backward_p1_f32src.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # no packed-FP32 (v_pk_*_f32) instruction selection in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for %s" % src)
    return obj


def _stale(src: str) -> bool:
    """Whether src's object is older than src or any header it may include."""
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")] + \
        [os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include"))]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(f) > t for f in deps)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (or, with ``incremental``, those whose object is
    older than the source or a header) and link libattnres.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = [s for s in SOURCES if not incremental or _stale(s)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, len(todo))) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv[1:])
