"""Build ``libmoe4.so`` (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_moe_expert_amd.build [-v]

Each ``csrc/*.hip`` file is compiled on its own (kernels are launched from the file
that defines them, so no relocatable device code is needed), then linked into
``bit_moe_expert_amd/libmoe4.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "moe4")
LIB_PATH = os.path.join(HERE, "libmoe4.so")

SOURCES = ["abi.hip", "route.hip", "permute.hip", "prepack.hip", "ffn_decode.hip", "ffn_prefill.hip", "ffn_prefill_fp8.hip", "combine.hip", "norm.hip", "quant.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are kept off: hipcc is told not to form them from plain
# float code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        ln for ln in (p.stdout + p.stderr).splitlines()
        if "packed-fp32-ops' is not a recognized feature" not in ln
    )
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libmoe4.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    shutil.move(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
