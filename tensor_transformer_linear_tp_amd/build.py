"""Build libtpshard.so for gfx950 in-tree with hipcc.

Every HIP/C++ source under csrc/ is compiled to an object under _build/ (in
parallel) and linked into ``libtpshard.so`` next to this file.  The library
depends only on the HIP runtime; it has no torch types in its interface.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libtpshard.so")
# Measurement helper (MFMA-only calibration kernel), a library of its own: not the method.
CALIB_PATH = os.path.join(PKG_DIR, "libtpcalib.so")
CALIB_SOURCES = ["calib_mfma.hip"]
ARCH = "gfx950"

SOURCES = ["abi.cpp", "gemm_bf16.hip", "gemm_f32.hip", "elementwise.hip", "embedding.hip", "attention.hip",
           "attention_bwd.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # Packed fp32 VALU ops stay off (the compiler would otherwise form them
    # from ordinary float code).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtpshard)")


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc, *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature name; that note is harmless.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l).strip()
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs and verbose:
        print(msgs, flush=True)
    return obj


def _link(objs, path: str, hipcc: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile and link libtpshard.so (and the calibration library libtpcalib.so);
    returns the path of libtpshard.so.  Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, hipcc, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH, hipcc)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_PATH, hipcc)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
