"""Build the fp4rollout shared library (libfp4rollout.so) for gfx950, in-tree.

    python -m fp4_quantized_diffusion_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
generation disabled; the quantization kernels additionally with
-ffp-contract=off (their rounding is defined operation by operation) and
correctly-rounded fp32 division. The C-ABI layer is plain host C++.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfp4rollout.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-fhip-fp32-correctly-rounded-divide-sqrt", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "lora.hip": ["-ffp-contract=off"],
    "nft.hip": ["-ffp-contract=off"],
    "gemm_mx.hip": [],
    "gemm_nv.hip": [],
    "euler.hip": [],
    "reward_select.hip": [],
}
HOST_SOURCES = ["abi.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n  " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose=False, jobs=8):
    """Compile every source and link libfp4rollout.so next to this file."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds, objs = [], []
    for src, extra in HIP_SOURCES.items():
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmds.append([HIPCC, *HIP_COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmds.append(["g++", "-std=c++17", "-O2", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra",
                     "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}",
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    shutil.move(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
