"""Build libmxfp8moe.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m moe_expert_grouped_group_amd.build

Each source is compiled by hipcc into an object under ``_build/`` (in
parallel), then linked into ``moe_expert_grouped_group_amd/libmxfp8moe.so``.
Packed-fp32 instructions are disabled for the device code
(``-target-feature -packed-fp32-ops``), and so is the atomic optimizer.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp8moe.so")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip"]
ARCH = "gfx950"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # atomics stay single instructions: the atomic optimizer would
            # turn the GEMM's tile-counter fetch into a wave-wide form that
            # waits for every outstanding memory operation right after it
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-Wno-unused-command-line-argument", "-Wno-inline-asm",
            "-I", os.path.join(ROOT, "include")]


def build(verbose=False):
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc, "-x", "hip"] + cmd[1:]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
