"""Build the gfx950 attention library (libattn_mi355x.so) in-tree with hipcc.

Usage: python -m attention_online_softmax_attn_amd.build   (or call build())
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn_mi355x.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["fwd_kernels.hip", "decode_kernels.hip", "bwd_kernels.hip", "bwd_dq.hip", "attn_abi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall",
]


# Per-source scheduling: the dK/dV kernel runs one wave per SIMD, so its LDS
# operand reads must be issued well ahead of the MFMAs that use them and the
# exponentials interleaved with independent MFMAs; the ILP-maximising machine
# scheduler does that, the default (occupancy-driven) one sinks every read next
# to its use.  The dQ kernel (bwd_dq.hip) measured faster with the default.
SOURCE_FLAGS = {
    "bwd_kernels.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _compile(src: str, objdir: str = OBJDIR, defines=()) -> str:
    os.makedirs(objdir, exist_ok=True)
    out = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = SOURCE_FLAGS.get(src, [])
    cmd = [HIPCC, *FLAGS, *extra, *[f"-D{d}" for d in defines], *lang, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return out


def build(verbose: bool = False, lib: str = LIB, objdir: str = OBJDIR, defines=()) -> str:
    """Compile every source for gfx950 and link the shared library.  Always rebuilds.

    ``defines`` (NAME=VALUE strings) override the kernels' compile-time tile
    choices; the default library is built without any."""
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
