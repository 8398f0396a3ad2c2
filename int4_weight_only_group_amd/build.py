"""Build libw4.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m int4_weight_only_group_amd.build        # or: from ... import build; build()

Objects go to <repo>/_build, the library to int4_weight_only_group_amd/libw4.so.
Always recompiles every source (no staleness tracking), in parallel.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-f32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # explicit floating-point contract: fused multiply-adds allowed, denormals kept
    "-ffp-contract=fast", "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[hipcc, *HIPCC_FLAGS, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(8, len(cmds))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for cmd, fut in zip(cmds, [ex.submit(_run, c) for c in cmds]):
            if verbose:
                print(" ".join(cmd))
            fut.result()
    tmp = LIB + ".tmp"
    link = [hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link))
    _run(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
