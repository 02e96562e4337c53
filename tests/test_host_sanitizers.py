"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every source of libkda.so with the sanitizers on the host side only
(each -fsanitize flag behind -Xarch_host: the gfx950 device code is the usual
one), links tests/host/abi_validation_driver.c against it with the same
sanitizers, and runs the driver: every call it makes is rejected on the host
or is a documented no-op, so nothing is launched and no GPU is needed.  Any
sanitizer report, or an unexpected status code, fails the test.  CPU only.
"""
import os
import shutil
import subprocess

import pytest

from kimi_delta_attention_chunked_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _clang():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    for p in (os.path.join(rocm, "llvm", "bin", "clang"), shutil.which("clang")):
        if p and os.path.exists(p):
            return p
    return None


@pytest.mark.skipif(_clang() is None or not os.path.exists(_build.hipcc()) and shutil.which("hipcc") is None,
                    reason="needs the ROCm toolchain (hipcc and its clang)")
def test_abi_validation_under_asan_ubsan(tmp_path):
    flags = [f for f in _build.HIPCC_FLAGS if f != "-Werror"] + SANITIZE + ["-g", "-O1"]
    procs, objs = [], []
    for src in _build.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        procs.append(subprocess.Popen([_build.hipcc(), *flags, "-c", os.path.join(_build.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    for p, src in zip(procs, _build.SOURCES):
        _, err = p.communicate()
        assert p.returncode == 0, "%s:\n%s" % (src, err[-3000:])
    lib = str(tmp_path / "libkda_san.so")
    subprocess.run([_build.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *SANITIZE, *objs, "-o", lib],
                   check=True, capture_output=True)
    exe = str(tmp_path / "abi_validation_driver")
    subprocess.run([_clang(), "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "host", "abi_validation_driver.c"),
                    lib, "-Wl,-rpath," + str(tmp_path), "-o", exe], check=True, capture_output=True)
    env = dict(os.environ)
    # The HIP runtime's own allocations outlive main; leak reports are about
    # it, not about this library's host code.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "abi validation under sanitizers: ok" in out
