"""Build libhs2.so (gfx950 HIP kernels + C-ABI shim) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-fp32 VALU
instruction selection disabled (-packed-fp32-ops), then linked into one shared
library next to this file.  ``python -m long_context_sparse_full_amd.build``
rebuilds it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libhs2.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "attn.hip", "select.hip", "bridge.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


# Per-source flags.  attn.hip: MFMA results in VGPRs rather than AGPRs, so the
# online-softmax rescale of the accumulators needs no AGPR round trips.
SOURCE_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, build_dir: str = BUILD_DIR, defines: tuple = (), extra: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, *[f"-D{d}" for d in defines], "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines: tuple = (), extra: tuple = ()) -> str:
    """Compile and link; `defines` are extra -D flags and `extra` extra compiler
    flags (compile-time tuning)."""
    build_dir = BUILD_DIR if out == LIB else os.path.join(os.path.dirname(out), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, tuple(defines), tuple(extra)), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
