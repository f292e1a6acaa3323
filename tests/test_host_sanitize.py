"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/host_sanitize/harness.cpp links the real kvevict.cpp
(validation, workspace layout and carving, table copies, call ordering)
against host stand-ins for the HIP runtime and for the kernel launchers,
which check every pointer a kernel would touch against the registered
allocations over the extent it indexes, and that a layer's arrays are
disjoint.  Built with g++ (no GPU code is involved)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "budgeted_decode_attention_amd", "csrc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    out = str(tmp_path_factory.mktemp("asan") / "kv_harness")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_sanitize", "harness.cpp"), os.path.join(CSRC, "kvevict.cpp"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def _env():
    env = dict(os.environ)
    # verify_asan_link_order=0: ASan need not be the first library loaded
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return env


def test_abi_host_code_is_clean_under_asan_and_ubsan(harness):
    r = subprocess.run([harness], capture_output=True, text=True, env=_env(), timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.strip().endswith("ok")
    assert r.stdout.count("scenario ") == 9


def test_harness_stops_on_an_out_of_bounds_extent(harness):
    r = subprocess.run([harness, "--short-input"], capture_output=True, text=True, env=_env(), timeout=300)
    assert r.returncode != 0
    assert "outside every allocation" in r.stderr
