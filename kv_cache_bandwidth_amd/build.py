"""Build the HIP library (libart.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libart.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit multiply-add fusion: the kernels write their fused
    # multiply-adds out, so every inlined copy of a computation rounds alike
    "-ffp-contract=off",
    # a wave's atomics here are issued by one lane on purpose; the optimizer's
    # wave-wide rewrite would read every result at once (a wait for all loads)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


# art_kernels.hip is compiled once per launch part (ART_PART, see the end of
# that file) so that the parts build in parallel; the objects, art_api.cpp and
# art_scratch.hip are then linked into the shared library.
PARTS = (0, 1, 2, 3)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = os.path.join(ROOT, "_build")
    os.makedirs(out, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for part in PARTS:
        obj = os.path.join(out, f"art_kernels_part{part}.o")
        jobs.append((obj, [hipcc, *flags, *inc, f"-DART_PART={part}", "-c",
                           os.path.join(CSRC, "art_kernels.hip"), "-o", obj]))
    api = os.path.join(out, "art_api.o")
    jobs.append((api, [hipcc, *flags, *inc, "-c", os.path.join(CSRC, "art_api.cpp"), "-o", api]))
    scr = os.path.join(out, "art_scratch.o")
    jobs.append((scr, [hipcc, *flags, *inc, "-c", os.path.join(CSRC, "art_scratch.hip"), "-o", scr]))
    procs = []
    for obj, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errors = []
    for cmd, pr in procs:
        _, err = pr.communicate()
        if pr.returncode != 0:
            errors.append(f"{' '.join(cmd[-4:])}: {err[-3000:]}")
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    link = [hipcc, *HIPCC_FLAGS, *[obj for obj, _ in jobs], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{r.stderr[-4000:]}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
