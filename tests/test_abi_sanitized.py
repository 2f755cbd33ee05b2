"""The C ABI's argument checking under AddressSanitizer and UndefinedBehaviorSanitizer.

The host code of the entry points (api.hip, block_api.hip) is compiled again with the
sanitizers on its host side only (the device code is unchanged) and linked with the other
objects of the library build and tests/abi_sanitize_driver.cpp, which makes every rejected
call of the ABI: out-of-bounds accesses, signed overflow and other undefined behaviour in
the validation and size arithmetic abort the driver.  No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "self_modifying_memory_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_SOURCES = ("api.hip", "block_api.hip")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_abi_checks_under_address_and_ub_sanitizers(tmp_path):
    from self_modifying_memory_amd import build as B
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    others = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in B.SOURCES if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("library objects not built (python -m self_modifying_memory_amd.build)")
    objs = []
    for src in HOST_SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".san.o"))
        cmd = [hipcc, *B.HIP_FLAGS, *SAN, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    # the driver is plain host C++ (g++, sanitized); the link takes the device code along
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        "-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_driver")
    cmd = [hipcc, f"--offload-arch={B.ARCH}", *SAN, drv, *objs, *others, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert "all argument checks as expected" in r.stdout
