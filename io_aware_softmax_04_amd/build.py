"""Build libiofa.so (the C-ABI library and its gfx950 kernels) in-tree.

    python -m io_aware_softmax_04_amd.build

Compiles every HIP source for gfx950 with hipcc and links one shared
library at io_aware_softmax_04_amd/_lib/libiofa.so, plus two measurement
helpers that are not part of it: the standalone MFMA-ceiling program
_lib/mfma_ceiling and the shader-clock probe _lib/libiofa_clock.so.  Packed fp32 vector
instructions are disabled for all device code.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(OUT_DIR, "libiofa.so")
CEILING = os.path.join(OUT_DIR, "mfma_ceiling")
CEILING_SOURCE = "mfma_ceiling.hip"
CLOCK = os.path.join(OUT_DIR, "libiofa_clock.so")
CLOCK_SOURCE = "clock_probe.hip"

SOURCES = ["fa_api.cpp", "fa_fwd_gfx950.hip", "fa_naive_gfx950.hip", "fa_merge_gfx950.hip",
           "fa_softmax_gfx950.hip", "fa_bwd_gfx950.hip", "fa_fwd_fp8_gfx950.hip",
           "fa_scratch_gfx950.hip"]

ARCH = "gfx950"
COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libiofa.so)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; its warning is noise
    lines = [ln for ln in proc.stdout.splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in ln]
    return proc.returncode, "\n".join(lines)


def build(verbose=False, extra_flags=()):
    """Compile and link; returns the path of the shared library."""
    cc = hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [cc, *COMMON, *extra_flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        rc, out = _run(cmd)
        return src, obj, rc, out, cmd

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for src, _, rc, out, cmd in results:
        if verbose or rc != 0:
            sys.stderr.write(f"[build] {' '.join(cmd)}\n{out}\n")
        if rc != 0:
            raise RuntimeError(f"compiling {src} failed:\n{out}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[r[1] for r in results], "-o", tmp]
    rc, out = _run(cmd)
    if rc != 0:
        raise RuntimeError(f"linking libiofa.so failed:\n{out}")
    os.replace(tmp, LIB)
    tmp = CEILING + ".tmp"
    cmd = [cc, "-std=c++17", "-O3", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", *extra_flags, os.path.join(CSRC, CEILING_SOURCE),
           "-o", tmp]
    rc, out = _run(cmd)
    if rc != 0:
        raise RuntimeError(f"building mfma_ceiling failed:\n{out}")
    os.replace(tmp, CEILING)
    tmp = CLOCK + ".tmp"
    cmd = [cc, *COMMON, *extra_flags, "-shared", "-x", "hip", os.path.join(CSRC, CLOCK_SOURCE),
           "-o", tmp]
    rc, out = _run(cmd)
    if rc != 0:
        raise RuntimeError(f"building libiofa_clock.so failed:\n{out}")
    os.replace(tmp, CLOCK)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
