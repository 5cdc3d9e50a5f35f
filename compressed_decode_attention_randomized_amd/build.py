"""Builds libkvq.so in-tree for gfx950 with hipcc.

    python -m compressed_decode_attention_randomized_amd.build [--jobs N]

Every HIP source is compiled with packed-FP32 instruction selection switched
off (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")
ARCH = "gfx950"

DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics", "-ffp-contract=fast",
                # matrix-core accumulators stay in VGPRs (no AGPR round trips around VALU rescaling)
                "-mllvm", "-amdgpu-mfma-vgpr-form",
                # one-lane LDS counter claims stay one atomic whose answer is read where the code reads it
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; libkvq needs ROCm's hipcc to build")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), *DEVICE_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    build(args.jobs)
    return 0


if __name__ == "__main__":
    sys.exit(main())
