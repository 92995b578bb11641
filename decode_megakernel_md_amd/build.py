"""Builds libmd.so (the gfx950 megakernel library) in place.

The kernel source is compiled twice: the 8-row build (decode up to 8
sequences, and the verify step) and the 64-row build (decode up to 64
sequences, kernel md_megakernel_w64); the host code picks one per model by
its max_batch."""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libmd.so")
CSRC = os.path.join(HERE, "csrc")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# 64-row build: matrix-core accumulators in ordinary vector registers (its
# stream holds four times the accumulators; in the accumulation registers
# they would be copied back and forth)
WIDE_FLAGS = ["-DMD_MAXB=64", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building libmd.so failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stderr


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include")]
    kern = os.path.join(CSRC, "md_kernel.hip")
    with tempfile.TemporaryDirectory(prefix="md_build_") as tmp:
        objs = [os.path.join(tmp, n) for n in ("k8.o", "k64.o", "host.o")]
        jobs = [
            ["hipcc", *HIPCC_FLAGS, *inc, "-c", kern, "-o", objs[0]],
            ["hipcc", *HIPCC_FLAGS, *WIDE_FLAGS, *inc, "-c", kern, "-o", objs[1]],
            ["hipcc", *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, "md_host.cpp"), "-o", objs[2]],
        ]
        with ThreadPoolExecutor(3) as ex:
            logs = list(ex.map(_run, jobs))
        logs.append(_run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", SO + ".tmp"]))
    if verbose:
        print("\n".join(logs))
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
