"""Build libbdstep.so (all HIP sources, gfx950) in-tree with hipcc.

Usage: python -m block_diffusion_lm_router_amd.build [--verbose]
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbdstep.so")
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU forms stay off: the compiler then never emits v_pk_{add,mul,fma}_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libbdstep")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose=False, jobs=None):
    """Compile every .hip source and link libbdstep.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON, "-c", src, "-o", obj])

    def run(cmd):
        res = subprocess.run(cmd, capture_output=True, text=True)
        return cmd, res

    jobs = jobs or min(8, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        for cmd, res in pool.map(run, cmds):
            noise = [ln for ln in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in ln]
            if verbose or res.returncode != 0:
                print(" ".join(cmd))
                if noise:
                    print("\n".join(noise))
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {cmd[-3]}")
    tmp = LIB + ".tmp"
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        print(res.stderr)
        raise RuntimeError("link of libbdstep.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
