"""The host side of the C ABI under sanitizers (no GPU): tests/sanitize_abi.cpp
drives every entry point's validation, workspace sizing and launch decisions,
with the kernel launchers, the HIP runtime calls and the rocBLAS calls stubbed,
built with g++ together with csrc/api.cpp and csrc/normal_api.cpp under
AddressSanitizer + UndefinedBehaviorSanitizer.  (mla_decode_latent_noalloc's
host code needs the HIP compiler for its device array; its size check is
covered through the built library by test_abi_cpu.py.)"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "mla_latent_kv_amd", "csrc")
SOURCES = [os.path.join(HERE, "sanitize_abi.cpp"), os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "normal_api.cpp")]


def test_abi_host_code_clean_under_address_and_undefined_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("g++ or the HIP headers not available")
    exe = str(tmp_path / "sanitized_abi")
    build = subprocess.run([cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                            "-I/opt/rocm/include", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            *SOURCES, "-o", exe], capture_output=True, text=True)
    if build.returncode != 0:
        if "libasan" in build.stderr or "libubsan" in build.stderr:
            pytest.skip("sanitizer runtime not installed: " + build.stderr.strip()[:200])
        raise AssertionError(build.stderr[-4000:])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=1"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr
