"""Build the native libraries in-tree.

``libmt.so``      : the C-ABI training-step library (HIP kernels for gfx950 and
                    the host runtime), from ``csrc/*.hip`` and ``csrc/*.cpp``.
``libmtsynth.so`` : the seeded synthetic-input generator (plain C).

Every call recompiles. Objects are compiled in parallel.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 ops stay off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-fopenmp", "-Wall", "-ffp-contract=off",
              "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build_synth(verbose: bool = False) -> str:
    src = os.path.join(CSRC, "synth", "synth.c")
    out = os.path.join(HERE, "libmtsynth.so")
    tmp = out + ".tmp"
    _run(["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_mt(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    include = os.path.join(ROOT, "include")
    hip_srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cpp_srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    if not hip_srcs and not cpp_srcs:
        raise RuntimeError("no sources under " + CSRC)
    jobs = jobs or max(1, min(16, os.cpu_count() or 1))

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [HIPCC, *HIP_FLAGS, f"-I{include}", f"-I{CSRC}", "-c", src, "-o", obj]
        else:
            cmd = ["g++", *HOST_FLAGS, "-march=x86-64-v3", f"-I{include}", f"-I{CSRC}",
                   "-c", src, "-o", obj]
        _run(cmd)
        if verbose:
            print("compiled", os.path.basename(src), flush=True)
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, hip_srcs + cpp_srcs))
    out = os.path.join(HERE, "libmt.so")
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
          "-fopenmp", "-lpthread", f"-L{ROCM}/lib", "-lamdhip64"])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_all(verbose: bool = False):
    build_synth(verbose)
    return build_mt(verbose)


if __name__ == "__main__":
    build_all(verbose=True)
