"""Build libw4a4.so in-tree with hipcc for gfx950.

Usage: python -m w4a4_gemm_lora_amd.build   (or call build()).
Every HIP translation unit is compiled with packed-fp32 instructions
disabled; the library links only against the HIP runtime.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libw4a4.so")
PEAKS_OUT = os.path.join(PKG, "libw4a4_peaks.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "graph.cpp", "quantize.hip", "gemm.hip", "noalloc.hip"]
# measurement-only microbenchmarks (attainable peaks), a library of their own
PEAKS_SOURCES = ["peaks.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, err))
    return err


def _objects(sources):
    objs, cmds = [], []
    for src in sources:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC] + COMMON + lang + ["-c", path, "-o", obj])
        objs.append(obj)
    return objs, cmds


def _link(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libw4a4.so (the layer)
    and libw4a4_peaks.so (the peak microbenchmarks); returns libw4a4.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, cmds = _objects(SOURCES)
    pobjs, pcmds = _objects(PEAKS_SOURCES)
    with ThreadPoolExecutor(max_workers=min(4, len(cmds) + len(pcmds))) as ex:
        for msg in ex.map(_run, cmds + pcmds):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    _link(objs, OUT)
    _link(pobjs, PEAKS_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
