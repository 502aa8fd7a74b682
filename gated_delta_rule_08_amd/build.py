"""Build libgdr.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m gated_delta_rule_08_amd.build``.  Every call recompiles
all sources; translation units compile in parallel.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdr.so")
ARCH = os.environ.get("GDR_OFFLOAD_ARCH", "gfx950")

SOURCES = ["gdr_api.hip", "decode.hip", "prefill_f32.hip", "prefill_bf16.hip", "backward.hip",
           "noalloc.hip"]

HIPFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # Packed fp32 instructions stay off in all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc()] + HIPFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = []
        for s in SOURCES:
            obj = os.path.join(out_dir, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, os.path.join(CSRC, s), obj))
        for f in futs:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
