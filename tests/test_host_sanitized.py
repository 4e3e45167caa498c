"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (the C ABI: argument, overlap and workspace checks, the device check)
and packer.cpp (the offline packers) are compiled with -fsanitize=address,
undefined and linked against a fake HIP runtime (tests/host_sanitize), which
reports a device of a chosen architecture and records launches instead of
running kernels.  The driver calls every entry point on heap buffers of
exactly the documented sizes.  It also forces the architecture check to fail:
the pages' loader refuses unsupported GPU generations at load time
(mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch Nunchaku
4-Bit-Quantisierung", section "Hardware-Unterstützung"), and so must every
device entry point here.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_diffusion_transformer_svdq_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("san") / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HERE,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "packer.cpp"),
           os.path.join(HERE, "fake_runtime.cpp"), os.path.join(HERE, "driver.cpp"), "-o", out, "-lpthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return out


def _run(driver, mode, **env):
    e = dict(os.environ)
    e.update(ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    e.update(env)
    return subprocess.run([driver, mode], capture_output=True, text=True, env=e, timeout=300)


def test_host_code_clean_under_sanitizers(driver):
    res = _run(driver, "full")
    assert res.returncode == 0, res.stdout + res.stderr[-6000:]
    assert "host checks passed" in res.stdout


def test_forced_architecture_mismatch(driver):
    res = _run(driver, "arch-mismatch", FAKE_GFX_ARCH="gfx942")
    assert res.returncode == 0, res.stdout + res.stderr[-6000:]


def test_no_device(driver):
    res = _run(driver, "no-device", FAKE_DEVICE_COUNT="0")
    assert res.returncode == 0, res.stdout + res.stderr[-6000:]
