"""The C ABI's host layer (argument validation, workspace layout, launch
parameters) built with AddressSanitizer and UndefinedBehaviorSanitizer and run
through its boundary cases, without a GPU.

The kernel launchers are replaced by host stand-ins (tests/host_sanitize/
launch_stubs.cpp) that check every buffer extent a kernel would touch against
the buffers the caller passed; tests/host_sanitize/boundary_driver.cpp runs good
and bad calls of every entry point and checks each status and launch count.
A second run plants a caller mistake (a workspace shorter than claimed) that
the stand-ins must catch.
"""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("host_sanitize") / "boundary_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "mla_latent_decode_absorbed_amd", "csrc"), "-I" + HERE,
           os.path.join(ROOT, "mla_latent_decode_absorbed_amd", "csrc", "mla_api.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "boundary_driver.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return out


def _run(driver, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([driver, *args], capture_output=True, text=True, env=env, timeout=120)


def test_boundary_cases_clean_under_sanitizers(driver):
    res = _run(driver)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "0 check failures, 0 extent failures" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr


def test_planted_short_workspace_is_caught(driver):
    res = _run(driver, "--plant-short-workspace")
    assert res.returncode == 1, res.stdout + res.stderr[-2000:]
    assert "ws_o" in res.stderr and "outside every registered buffer" in res.stderr
