"""Build libfa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

hipcc compiles each HIP source for --offload-arch=gfx950 only and links one
shared library next to this file. Packed fp32 VALU instructions are turned
off for device code (-packed-fp32-ops).
"""

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_f32.hip", "fa_bwd.hip", "fa_decode.hip",
           "fa_clock.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc_path():
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False, extra_flags=()):
    """Compile every source and link libfa.so; always rebuilds."""
    hipcc = hipcc_path()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
