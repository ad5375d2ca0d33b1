"""Build libfa.so (the gfx950 attention kernels and their C ABI) in-tree.

Every HIP translation unit is compiled by hipcc for gfx950 only, with packed
fp32 instruction generation disabled, then linked into one shared library
next to this file.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_wide.hip", "fa_bwd.hip", "fa_bwd_wide.hip", "fa_decode.hip", "fa_fp8.hip",
           "fa_f32.hip", "fa_noalloc.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    # no packed-fp32 (v_pk_*_f32) instructions in generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax rescale and the dS / P packing
    # read and write them with vector ALU ops, which cannot address AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", *COMMON_FLAGS, os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", LIB + ".tmp",
           "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
