"""Build libmc2.so for gfx950 with hipcc (in-tree, so the library travels with the tree).

Every HIP and C++ source under csrc/ is compiled to an object in parallel and
linked into ``comm_matmul_tensor_amd/libmc2.so``.  Objects go to ``_build/``.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "libmc2")
LIB = os.path.join(HERE, "libmc2.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instructions are disabled for all device code; fp32 division
# and square root stay correctly rounded (hipcc's default) and no fast-math.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", f"-I{os.path.join(ROOT, 'include')}",
          f"-I{CSRC}", "-fno-fast-math", "-ffp-contract=off"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = []
    name = os.path.basename(src)
    if name.startswith("gemm_"):
        # MFMA accumulators in VGPRs: the AGPR form made the register allocator
        # rotate accumulators through copies inside the main loop.
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    elif name == "gemm256.hip":
        # 256 accumulators per lane: AGPR form; and full unrolling of the
        # 64-MFMA half steps, which exceed the default unroll limit
        extra = ["-mllvm", "-pragma-unroll-threshold=1000000"]
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + extra + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip"] + COMMON + DEVICE_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
