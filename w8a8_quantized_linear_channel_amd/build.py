"""Build libq8.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled to an object under _build/ (in
parallel), then linked into w8a8_quantized_linear_channel_amd/libq8.so.
Always rebuilds: the build is the check that the sources compile.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq8.so")

ARCH = "gfx950"
COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Device code: no fast-math, correctly rounded fp32 division (the default),
# denormals kept, and the packed-fp32 instructions switched off.
HIP_ONLY = [
    f"--offload-arch={ARCH}",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libq8)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    objs = []
    cmds = []
    for f in srcs:
        obj = os.path.join(BUILD, f + ".o")
        objs.append(obj)
        flags = COMMON + HIP_ONLY if f.endswith(".hip") else COMMON + ["-D__HIP_PLATFORM_AMD__"]
        lang = ["-x", "hip"] if f.endswith(".hip") else []
        cmds.append([cc] + lang + flags + ["-c", os.path.join(CSRC, f), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
