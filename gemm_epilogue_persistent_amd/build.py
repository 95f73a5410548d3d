"""Build libgemm_mi355x.so (the C ABI + gfx950 kernels) in-tree with hipcc.

Every unit is compiled for gfx950 only. Packed-fp32 VALU instructions are disabled
(-packed-fp32-ops) for all device code. The atomic optimizer is off: it rewrites the
dynamic schedule's single-lane tile claim into a per-wave form that waits for the result
right away instead of where it is used.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgemm_mi355x.so")
# one unit per (operand type, epilogue kind, varlen mode) family of kernels
UNITS = ["plan.cpp", "gemm_api.hip"] + [
    f"inst_{op}_{fam}.hip" for op in ("f16", "bf16", "fp8") for fam in ("fwd", "vm", "vk", "dact", "dact_vm")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-Wno-unused-command-line-argument"]


PROBE_SRC = os.path.join(HERE, "measure", "mfma_probe.hip")
PROBE_LIB = os.path.join(HERE, "measure", "libmfma_probe.so")


def _compile(unit, verbose):
    src = os.path.join(CSRC, unit) if not os.path.isabs(unit) else unit
    obj = os.path.join(BUILD, os.path.basename(unit) + ".o")
    cmd = [hipcc()] + flags() + ["-c", src, "-o", obj]
    if unit.endswith(".cpp"):  # host-only C++ (no HIP call, no device code)
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {unit}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(UNITS), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), UNITS + [PROBE_SRC]))
    probe_obj = objs.pop()
    # the GEMM library, and the benchmark's MFMA probe in a library of its own
    for lib, parts in ((LIB, objs), (PROBE_LIB, [probe_obj])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + parts
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
