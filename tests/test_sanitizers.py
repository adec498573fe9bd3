"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code (CPU).

gcc builds, with -fsanitize=address,undefined (undefined behaviour aborts):
  * the oracle (oracle/ccl_oracle.c);
  * libccl's host side -- every entry point's argument checks, launch
    resolution and the reshard planner (csrc/ccl_api.cpp, csrc/ccl_plan.cpp)
    -- with the kernel launches replaced by stand-ins that stop the process
    if reached (tests/host_only_stubs.cpp).
The oracle pins and the host ABI / planner tests then run in a child Python
with the ASan runtime preloaded and both libraries swapped for the
sanitized builds.  Any sanitizer report fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "collective_communication_plane_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1", "-fno-fast-math", "-ffp-contract=off"]

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import oracle
oracle._LIB = {orc!r}
from collective_communication_plane_amd import ccl
ccl._LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                      {abi!r}, {pins!r},
                      "-k", "not plain_c_client and not bench_refuses"]))
"""


def _libasan() -> str:
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's ASan runtime is not installed")
    return p


@pytest.mark.timeout(900)
def test_host_code_and_oracle_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc not available")
    hip_inc, hip_lib = "/opt/rocm/include", "/opt/rocm/lib"
    if not os.path.exists(os.path.join(hip_lib, "libamdhip64.so")):
        pytest.skip("HIP runtime headers/library not available")
    asan = _libasan()
    orc = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", *SAN, "-shared", "-fPIC", "-o", orc,
                    os.path.join(ROOT, "oracle", "ccl_oracle.c")], check=True)
    lib = str(tmp_path / "libccl_host_san.so")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", hip_inc,
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-shared", "-fPIC",
                    os.path.join(CSRC, "ccl_api.cpp"), os.path.join(CSRC, "ccl_plan.cpp"),
                    os.path.join(ROOT, "tests", "host_only_stubs.cpp"),
                    "-L", hip_lib, "-lamdhip64", f"-Wl,-rpath,{hip_lib}", "-Wl,--no-undefined",
                    "-o", lib], check=True)
    tests = os.path.join(ROOT, "tests")
    code = CHILD.format(root=ROOT, tests=tests, orc=orc, lib=lib,
                        abi=os.path.join(tests, "test_host_abi.py"),
                        pins=os.path.join(tests, "test_oracle_pins.py"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=840)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout, out[-3000:]
    print(r.stdout.strip().splitlines()[-1])
