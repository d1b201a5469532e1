"""The C ABI's argument validation built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, g++; no GPU).  The driver
(tests/sanitize/abi_validation_driver.cpp) calls every entry point over a
grid of extreme sizes, bad head dimensions, dtypes, scales and pointers,
with the kernel launchers replaced at link time by stand-ins that check
what validation lets through and never touch a device."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "io_aware_softmax_04_amd")
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
KERNEL_OBJECTS = ["fa_fwd_gfx950.o", "fa_naive_gfx950.o", "fa_merge_gfx950.o",
                  "fa_softmax_gfx950.o", "fa_bwd_gfx950.o", "fa_fwd_fp8_gfx950.o",
                  "fa_scratch_gfx950.o"]
LAUNCHERS = ["_ZN4iofa12launch_fusedERKNS_7FwdArgsE",
             "_ZN4iofa20launch_fused_partialERKNS_7FwdArgsEiPfS3_",
             "_ZN4iofa12launch_mergeERKNS_9MergeArgsE",
             "_ZN4iofa12launch_naiveERKNS_9NaiveArgsE",
             "_ZN4iofa14launch_softmaxERKNS_11SoftmaxArgsE",
             "_ZN4iofa10launch_bwdERKNS_7BwdArgsE",
             "_ZN4iofa10launch_fp8ERKNS_7Fp8ArgsE",
             "_ZN4iofa15scratch_addressEPPv",
             "_ZN4iofa15softmax_x_readsERKNS_11SoftmaxArgsE"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert proc.returncode == 0, f"{' '.join(cmd)}\n{proc.stdout[-4000:]}"
    return proc.stdout


def test_validation_is_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    if not all(os.path.exists(os.path.join(OBJ, o)) for o in KERNEL_OBJECTS):
        import __graft_entry__
        __graft_entry__.build()
    flags = ["-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "driver.o", "driver"))
    _run(["g++", *flags, "-c", os.path.join(CSRC, "fa_api.cpp"), "-o", api_o])
    _run(["g++", *flags, "-c", os.path.join(ROOT, "tests", "sanitize",
                                            "abi_validation_driver.cpp"), "-o", drv_o])
    wraps = [f"-Wl,--wrap={s}" for s in LAUNCHERS]
    _run(["g++", *SAN, drv_o, api_o, *(os.path.join(OBJ, o) for o in KERNEL_OBJECTS), *wraps,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    out = _run([exe], env=env, timeout=600)
    print(out.strip())
    assert "failures 0" in out and "runtime error" not in out
