"""Build libbdstep.so (all HIP sources, gfx950) in-tree with hipcc.

Usage: python -m block_diffusion_lm_router_amd.build [--verbose]
"""

import concurrent.futures
import os
import re
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


# The compiler's per-kernel resource remarks are read back after each compile: no kernel may
# use scratch memory (a register spill to memory inside a streaming loop), and the GEMM
# kernels, launched on the assumption of two 8-wave blocks per CU, must keep 4 waves per SIMD
# (at most 128 VGPRs).  HIP's second launch bound is a minimum of waves per SIMD, not of
# blocks per CU, so the occupancy is checked here rather than requested there.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
MIN_WAVES_PER_SIMD = {"w4a16_packed_kernel": 4, "w4a16_down_resident_kernel": 4}


def check_resources(stderr):
    """Problems found in the kernel-resource-usage remarks of one compile (empty if none)."""
    problems, name = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            problems.append(f"{name}: {m.group(1)} bytes of scratch per lane")
        m = re.search(r"remark:\s+Occupancy \[waves/SIMD\]: (\d+)", line)
        if m and name:
            for key, need in MIN_WAVES_PER_SIMD.items():
                if key in name and int(m.group(1)) < need:
                    problems.append(f"{name}: {m.group(1)} waves per SIMD, needs {need}")
    return problems


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
        cmds.append([hipcc, *COMMON, *RESOURCE_REMARKS, "-c", src, "-o", obj])

    def run(cmd):
        res = subprocess.run(cmd, capture_output=True, text=True)
        return cmd, res

    jobs = jobs or min(8, os.cpu_count() or 1)
    problems = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        for cmd, res in pool.map(run, cmds):
            noise = [ln for ln in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln]
            if verbose or res.returncode != 0:
                print(" ".join(cmd))
                if noise:
                    print("\n".join(noise))
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {cmd[-3]}")
            problems += check_resources(res.stderr or "")
    if problems:
        raise RuntimeError("kernel resources out of bounds:\n  " + "\n  ".join(problems))
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
