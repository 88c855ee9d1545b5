"""Compile libpkv.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m paged_kv_cache_325_amd.build [-v]

Each ``csrc/*.hip`` file (hipcc) and each host-only ``csrc/*.cpp`` file (g++)
is compiled to an object under ``_build/`` in parallel, then linked into
``paged_kv_cache_325_amd/libpkv.so``.  Packed-fp32
VALU instructions are disabled for device code.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpkv")
    return exe


def gxx() -> str:
    exe = shutil.which("g++")
    if not exe:
        raise RuntimeError("g++ not found; it builds the host-only C++ sources of libpkv")
    return exe


# prefill.hip: no NaN reaches its max reductions (masked scores are -inf via
# an integer-compare select), so fmaxf needs no NaN canonicalisation; that
# halves the VALU work of the row max.  Infinities keep their meaning.
# decode.hip: the MFMA accumulators of the shared-prefix path stay in VGPRs
# (the default puts them in AGPRs, which count against the same per-SIMD
# register file and took the kernel from two waves per SIMD to one); the
# kernels without MFMA compile to the same code either way.
PER_FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"],
                  "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _flags():
    f = [
        f"--offload-arch={ARCH}",
        "-std=c++17",
        "-fPIC",
        "-O3",
        "-Wall",
        "-Wno-unused-function",
        f"-I{INCLUDE}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]
    return f


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = _flags()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *flags, *PER_FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose:
            sys.stderr.write(r.stderr)
        return obj

    def compile_host(src):
        # host-only C++ (the block manager): no device code, plain g++
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".host.o")
        cmd = [gxx(), "-std=c++17", "-fPIC", "-O2", "-Wall", f"-I{INCLUDE}", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    host_srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(host_srcs))) as ex:
        futs = [ex.submit(compile_one, s) for s in srcs] + [ex.submit(compile_host, s)
                                                          for s in host_srcs]
        objs = [f.result() for f in futs]
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
