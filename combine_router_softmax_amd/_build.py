"""Builds the gfx950 HIP library libmoe_mi355x.so in-tree with hipcc.

Each source is compiled to an object under _build/ (in parallel), then the
objects are linked into the shared library next to this file.  Every HIP
compile carries the packed-fp32 target-feature switch that keeps hipcc from
emitting packed fp32 arithmetic.

moe_ffn_mx.hip (the MXFP8 expert FFN) is compiled with LLVM's machine-sinking
pass switched off.  That pass moves instructions down into the block where
their results are next used.  In the MXFP8 K loop it moved the first slice's
MFMAs past the conditional loads of the step after next, and so past the
step's wait and barrier.  The wave then waited for the loads and for the LDS
fragment reads with no MFMA in flight, and issued all of the step's MFMAs back
to back afterwards.  Without the pass the loop keeps the interleave that its
scheduling barriers describe.  The bf16 loops keep it either way and are built
with the default passes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libmoe_mi355x.so"
SOURCES = ["moe_abi.cpp", "moe_route.hip", "moe_layout.hip", "moe_rows.hip", "moe_mxfp8.hip", "moe_ffn.hip", "moe_ffn_mx.hip",
           "moe_replica.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", str(PKG.parent / "include")]
EXTRA_FLAGS = {"moe_ffn_mx.hip": ["-mllvm", "-disable-machine-sink"]}


def _compile(src: str) -> Path:
    obj = BUILD / (Path(src).stem + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA_FLAGS.get(src, []), "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stderr or "").splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err)
    return obj


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
