"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU (no GPU):

- the CPU oracle (oracle/kq_oracle.c) and the input generator (synth/synth.c),
  compiled with gcc -fsanitize=address,undefined together with a driver that
  calls every exported function on exact-size buffers (tests/sanitize/);
- the host side of libkq.so: the library rebuilt with the sanitizers on its
  host code only (hipcc's -Xarch_host; device code unchanged) and a C driver
  that drives every entry point's argument checks, including sizes whose
  products overflow int64, and the host-only helpers.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), which
fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# sanitizers on the host pass only
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")


def run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), p.stdout[-4000:], p.stderr[-4000:])
    return p


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_synth")
    run(["gcc", "-std=c11", "-D_GNU_SOURCE", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-pthread",
         os.path.join(SAN, "oracle_synth_driver.c"), os.path.join(ROOT, "oracle", "kq_oracle.c"),
         os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm"])
    p = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    assert "ok" in p.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANG), reason="ROCm toolchain not found")
def test_library_host_checks_under_asan_ubsan(tmp_path):
    from mxfp4_activation_quantizer_amd import build as kqbuild
    lib = str(tmp_path / "libkq_san.so")
    flags = [f for f in kqbuild.HIP_FLAGS if f != "-O3"] + ["-O1", "-g"]
    run([HIPCC, *flags, *HOST_SAN, "-I", kqbuild.INCLUDE, "-I", kqbuild.CSRC, *kqbuild.sources(), "-o", lib])
    exe = str(tmp_path / "host_checks")
    run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-I", kqbuild.INCLUDE, os.path.join(SAN, "host_checks_driver.c"), "-L", str(tmp_path), "-lkq_san",
         "-Wl,-rpath," + str(tmp_path), "-o", exe])
    p = run([exe], env=ENV)
    assert "ok" in p.stdout
