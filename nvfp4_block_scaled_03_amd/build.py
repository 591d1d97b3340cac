"""Build libnvfp4moe.so for gfx950 with hipcc (in-tree).

    python -m nvfp4_block_scaled_03_amd.build [-v]

Every source under csrc/ is compiled for gfx950 only, in parallel, into
_build/, and linked into nvfp4_block_scaled_03_amd/libnvfp4moe.so.  Packed FP32
VALU instructions are disabled for device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnvfp4moe.so")
ARCH = "gfx950"
SOURCES = ["api.hip", "codec.hip", "align.hip", "prep.hip", "gemm.hip", "mx.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def build(verbose: bool = False, jobs: int = 8, out: str = LIB, defines=(), build_dir: str = BUILD) -> str:
    """Compile and link; ``defines`` are extra -D settings, ``out`` the library path."""
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *["-D" + d for d in defines], "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
