"""Build libcsa.so (the HIP kernels and their C ABI) for gfx950, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["abi.cpp", "compress.hip", "indexer.hip", "topk.hip", "mqa.hip", "mqa_wide.hip", "mx4.hip", "cache.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed-fp32 instructions are disabled for all device code
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]
# per-source additions: MFMA results go to VGPRs for the indexers (each
# epilogue reads every one of them; results in AGPRs cost one accvgpr read
# each) and for the wide attention kernel (its accumulator is rescaled by VALU
# code; in AGPRs the compiler keeps a second, VGPR copy of it every tile)
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {"indexer.hip": _VGPR_MFMA, "mx4.hip": _VGPR_MFMA, "mqa_wide.hip": _VGPR_MFMA}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 5) -> str:
    """Compile every source and link libcsa.so; always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
