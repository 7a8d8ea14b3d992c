"""Build libattn.so (HIP, gfx950) in-tree.

    python -m transformer_attention_03_amd.build

Compiles the library's sources under csrc/ with hipcc for gfx950 and links them into
transformer_attention_03_amd/libattn.so, and the memory-system floor probes that the
benchmark times beside the kernels (csrc/floors.hip) into libattn_floors.so.  Packed FP32
instructions are disabled (-packed-fp32-ops) for all device code.
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
LIB = os.path.join(PKG, "libattn.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["api.cpp", "decode.hip", "fwd.hip", "block_local.hip"]
FLOORS_SOURCE = "floors.hip"
FLOORS_LIB = os.path.join(PKG, "libattn_floors.so")
# per-source extra hipcc flags (none at present)
KERNEL_FLAGS = {}
ARCH = os.environ.get("TA03_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def compile_flags(extra=()):
    return ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in VGPRs: the softmax reads the score tiles directly
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function",
            "-Wno-unused-variable", "-Wno-unused-but-set-variable", *extra]


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(extra), *KERNEL_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-8000:]))
    if r.stderr.strip():
        # keep warnings visible (but the host pass's note about the packed-fp32 feature is noise)
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))
    os.replace(tmp, out)


def build(verbose: bool = True, extra=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + [FLOORS_SOURCE]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], FLOORS_LIB)
    if verbose:
        print("built", LIB, "and", FLOORS_LIB)
    return LIB


if __name__ == "__main__":
    build()
