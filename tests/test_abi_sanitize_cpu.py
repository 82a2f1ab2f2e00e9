"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp (argument validation, workspace sizing, device check, dispatch
counters) and the driver tests/abi_host_check.cpp are compiled with g++
-fsanitize=address,undefined and linked with the kernel objects of the
regular build. The driver calls every exported entry point with seeded
random combinations of null, aligned and misaligned pointers, in-range and
out-of-range enums and sizes up to 2^40, where no HIP device is visible (it
calls nothing when one is). Any out-of-bounds host access, signed overflow
or invalid shift in the host code fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "w4a8_rotated_quantized_amd")
BUILD = os.path.join(PKG, "_build")
KERNEL_OBJS = ["rq.o", "pack.o", "merge.o", "gemm_w4a4.o", "gemm_int.o", "gemm_w4a8.o", "gemm_f6.o"]
ROCM = "/opt/rocm"


def _missing():
    if not shutil.which("g++"):
        return "g++ not available"
    if not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        return "HIP headers not available"
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in KERNEL_OBJS):
        return "kernel objects not built (run the build first)"
    return None


@pytest.mark.skipif(_missing() is not None, reason=str(_missing()))
def test_abi_host_layer_under_sanitizers(tmp_path):
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
             f"-I{os.path.join(ROOT, 'include')}"]
    abi_o = str(tmp_path / "abi_san.o")
    drv_o = str(tmp_path / "check.o")
    exe = str(tmp_path / "abi_host_check")
    subprocess.run(["g++", *flags, "-c", os.path.join(PKG, "csrc", "abi.cpp"), "-o", abi_o], check=True)
    subprocess.run(["g++", *flags, "-c", os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", drv_o], check=True)
    subprocess.run(["g++", "-fsanitize=address,undefined", drv_o, abi_o,
                    *[os.path.join(BUILD, o) for o in KERNEL_OBJS],
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe], check=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert ("all ok" in r.stdout) or ("skipped" in r.stdout), out[-4000:]
