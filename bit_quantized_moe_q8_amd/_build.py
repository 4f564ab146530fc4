"""Build libpq.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["pq_api.cpp", "pq_selftest.cpp", "k_prep.hip", "k_matvec.hip", "k_matvec1.hip", "k_tile_q8.hip", "k_gemm.hip", "k_peak.hip"]

# No fast-math: the q8 rule needs correctly rounded fp32 division.  Packed
# fp32 VALU forms are disabled for all device code.
FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# The int8 MFMA tile converts every MFMA result with VALU instructions, which
# cannot read accumulation registers: results go straight to VGPRs (the
# mat-vec file holds the tile's body too, for the skewed-decode launch).
FILE_FLAGS = {"k_tile_q8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "k_matvec.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _stale(src: str, obj: str) -> bool:
    """The object is older than its source or any header of csrc/include."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".hpp")]
    deps.append(os.path.join(os.path.dirname(HERE), "include", "pq.h"))
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    if incremental and not _stale(src, obj):
        return obj
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source and link libpq.so (always rebuilds, unless
    `incremental`: then only sources older than their objects' inputs)."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
