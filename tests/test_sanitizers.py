"""The CPU oracle (oracle/moe_oracle.c) and the host-only slot pool
(csrc/pool_fake.cpp with the pool code of pool_core.h) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through every
entry point by tests/sanitize/driver.cpp; any report fails the run (no
recovery).  CPU only: gcc / g++, no GPU code in the build."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int4_weight_only_router_amd", "csrc")


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                    reason="needs gcc and g++")
def test_oracle_and_host_pool_clean_under_asan_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-g", "-O1"]
    obj = str(tmp_path / "oracle.o")
    exe = str(tmp_path / "driver")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-c",
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", obj] + san, check=True)
    subprocess.run(["g++", "-std=c++17", "-fopenmp", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
                    os.path.join(CSRC, "pool_fake.cpp"), obj, "-o", exe] + san, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="3")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized run clean" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
