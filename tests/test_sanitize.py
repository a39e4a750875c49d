"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two standalone drivers (sources in tests/sanitize/):
  * the C oracles built with gcc and both sanitizers, run on edge shapes;
  * the library (its host code built with both sanitizers, its device code
    as usual) linked into a driver that calls every entry point with
    arguments it must refuse before touching the device, and the workspace
    queries over edge and extreme sizes.  Nothing is launched (there is no
    GPU here: a call that got past the checks would fail at its launch), so
    this checks memory and arithmetic safety of the host paths; which check
    refuses what is tested in test_abi.py.
A sanitizer report aborts the driver (recovery off), failing the test.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_31_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "include")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
# each sanitizer flag directly after -Xarch_host: host code only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def test_oracles_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    srcs = [os.path.join(SAN, "oracle_driver.c")] + sorted(
        glob.glob(os.path.join(ROOT, "oracle", "*.c")))
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe] + srcs +
                   ["-lm", "-lpthread"])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0, out[-4000:]
    assert "0 failed check(s)" in out


def test_library_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + HOST_SAN
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [str(tmp_path / (os.path.basename(s)[:-4] + ".o")) for s in srcs]

    def compile_one(so):
        return _run([HIPCC] + flags + ["-c", "-o", so[1], so[0]])

    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        for rc, out in ex.map(compile_one, zip(srcs, objs)):
            assert rc == 0, out
    drv = str(tmp_path / "abi_driver.o")
    rc, out = _run([HIPCC, "-x", "c++", "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", ROCM_INCLUDE, "-D__HIP_PLATFORM_AMD__"] + HOST_SAN +
                   ["-c", "-o", drv, os.path.join(SAN, "abi_driver.cpp")])
    assert rc == 0, out
    exe = str(tmp_path / "abi_driver")
    rc, out = _run([HIPCC, "--offload-arch=gfx950"] + HOST_SAN + ["-o", exe, drv] + objs)
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0, out[-4000:]
    assert "0 call(s) not rejected" in out
