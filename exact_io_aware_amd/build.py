"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

Run as ``python -m exact_io_aware_amd.build``.  hipcc cross-compiles, so no
GPU is needed to build.  Each source is compiled to its own object in
parallel (the attention kernel's instances are split over four sources, one
per input type and head dimension), then the objects are linked.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
# The test build: the same kernels with their LDS filled with NaN before use
# (FA_POISON_LDS=1; csrc/fa_poison.h).  Only tests load it.
POISON_LIB = os.path.join(PKG, "libfa_poison.so")
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["fa_fwd_mfma_bf16_d128.hip", "fa_fwd_mfma_f16_d128.hip", "fa_fwd_mfma_bf16_d64.hip",
           "fa_fwd_mfma_f16_d64.hip", "fa_fwd_kernels.hip", "fa_bwd_kernels.hip", "fa_api.cpp",
           "fa_validate.cpp"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# The host pass does not know the packed-fp32 feature name; that note is
# harmless, everything else is shown.
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    return res.returncode, msgs


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16, len(SOURCES)))


def build(verbose: bool = False, poison: bool = False) -> str:
    """Compile libfa.so (poison: libfa_poison.so, the LDS-poisoning test
    build); returns its path.  Raises on a compiler error."""
    objdir = os.path.join(OBJDIR, "poison") if poison else OBJDIR
    lib_path = POISON_LIB if poison else LIB
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    defs = ["-DFA_POISON_LDS=1"] if poison else []

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        return src, obj, _run([hipcc(), *HIPCC_FLAGS, *defs, *inc, "-c",
                               os.path.join(CSRC, src), "-o", obj])

    objs, errors, notes = [], [], []
    with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for src, obj, (rc, msgs) in ex.map(compile_one, SOURCES):
            objs.append(obj)
            (errors if rc != 0 else notes).extend(msgs)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = lib_path + ".tmp"
    rc, msgs = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    notes.extend(msgs)
    if verbose and notes:
        print("\n".join(notes), file=sys.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, poison=True))
