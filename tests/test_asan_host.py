"""The library's host code (argument validation, status codes, per-thread messages) under
AddressSanitizer, on the CPU: the HIP sources are rebuilt with the host pass instrumented
(the device code is not; it is not run) and a plain C driver (tests/asan/abi_asan.c),
instrumented too, calls every entry point from four threads with arguments that are
rejected or are empty batches, so no call launches device work. A memory error aborts the
driver with a sanitizer report. The oracle is numpy code and needs no sanitizer."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_asan(tmp_path):
    from normalisation_dilated_conv1d_amd.build import HIP_FLAGS

    csrc = os.path.join(ROOT, "normalisation_dilated_conv1d_amd", "csrc")
    lib = tmp_path / "libdconv1d.so"
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    build = [HIPCC, *HIP_FLAGS, "-shared", *asan, "-g", f"-I{ROOT}/include", f"-I{csrc}",
             *sorted(glob.glob(os.path.join(csrc, "*.hip"))), "-o", str(lib)]
    r = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_asan"
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    link = [clang, "-std=c99", "-g", "-O1", "-fsanitize=address", "-fno-omit-frame-pointer",
            "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{ROCM}/include",
            os.path.join(ROOT, "tests", "asan", "abi_asan.c"), f"-L{tmp_path}", "-ldconv1d",
            f"-L{ROCM}/lib", "-lamdhip64", "-lpthread", f"-Wl,-rpath,{tmp_path}",
            f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    r = subprocess.run(link, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    # leak checking is off: the HIP runtime keeps process-lifetime allocations
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-5000:]
    assert "all checks passed" in r.stdout
