"""Build libcsa.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled with packed-fp32 instruction generation disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libcsa.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "compress.hip", "indexer.hip", "attend.hip", "attend_bwd.hip", "indexer_bwd.hip",
           "compress_bwd.hip"]
# Per-source extra flags.  attend.hip and indexer.hip keep their MFMA
# accumulators in VGPRs: the attention loops rescale the output accumulator
# conditionally and the score epilogues read every accumulator element, and
# with the accumulators in AGPRs the compiler copies them to VGPRs on every
# key tile.
EXTRA = {"attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = os.environ.get("CSA_OFFLOAD_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-O3", "-fPIC", "-std=c++17", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-Wall", "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = ["hipcc", *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(errs)))
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build() -> str:
    """Compile every HIP source and link libcsa.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    # rocBLAS serves the compressor backward's plain GEMMs (dx, dW)
    subprocess.check_call(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs,
                           "-L" + os.path.join(ROCM, "lib"), "-lrocblas",
                           "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
