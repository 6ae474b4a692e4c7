"""Build libhypic.so in-tree: hipcc, gfx950 only.

Compiles every HIP/C++ source under csrc/ to an object in <repo>/_build/ and
links them into linear_attention_state_chunked_amd/libhypic.so.  The
matrix-core rate probe (csrc/probe/) becomes its own libhypic_probe.so.
Always recompiles (the build check runs it on every call).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libhypic.so")
PROBE_OUT = os.path.join(PKG, "libhypic_probe.so")
PROBE_SOURCES = [os.path.join("probe", "mfma_probe.hip")]
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gdn_build.hip", "dense_engine.hip", "diag_build.hip", "compose.hip", "conv.hip", "seam.hip", "rope.hip", "kda_build.hip",
           "hypic_host.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 instructions disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build())
