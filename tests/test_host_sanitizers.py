"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): csrc/api.hip (argument checks, device check, plan choice,
last-error text) is compiled with the sanitizers on its host side only
(each -fsanitize= flag behind -Xarch_host, so no device code is
instrumented), linked with the unsanitized kernels and a driver
(tests/sanitize/abi_driver.cpp) that exercises every refusal path --
bad shapes, null and misaligned pointers, leading dimensions, workspace
sizes, the no-device answer -- and the diagnostics.  Any sanitizer report
fails the test."""

import os
import shutil
import subprocess

import pytest

from fine_grained_block_fp8_amd import build as fgbuild

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="HIP toolchain not installed")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    cc = fgbuild.hipcc()
    common = [a for a in fgbuild.COMMON if a != "-fPIC"]
    objs = []
    for src in fgbuild.sources():
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        flags = SAN if os.path.basename(src) == "api.hip" else []
        r = subprocess.run([cc, *common, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    r = subprocess.run([cc, "-x", "hip", *common, *SAN, "-c", os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([cc, f"--offload-arch={fgbuild.ARCH}", *SAN, drv, *objs, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # without a device the valid calls must answer FGFP8_ENODEV; with one, the
    # driver skips those expectations
    args = ["device"] if os.environ.get("FGFP8_SANITIZE_WITH_DEVICE") else []
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "all ABI checks passed" in r.stdout, out[-4000:]
