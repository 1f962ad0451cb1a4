"""Build libtwell.so (the HIP kernels + the C ABI) in-tree for gfx950.

    python -m activation_sparse_transformer_amd.build

Each ``csrc/*.hip`` is compiled by hipcc to an object under ``_build/`` (in
parallel), then linked into ``activation_sparse_transformer_amd/libtwell.so``.
Always rebuilds: it is the does-it-build check as well as the build.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtwell.so")
ARCH = "gfx950"

SOURCES = ["twell_api.hip", "gemm_bf16.hip", "gemm_f32.hip", "route.hip", "spmm.hip", "skinny.hip",
           "ell.hip", "backward.hip", "gate.hip"]

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off: every fp32 op is a plain VALU op
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[hipcc, *CFLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(8, len(cmds))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fvisibility=hidden", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
