"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs, each built with one compiler so that one sanitizer runtime
serves it: libwq's sources compiled with the sanitizers on the host side only
(the GPU code is built as usual and never launched), linked with
tests/sanitize/host_san.c, which runs the host packer, the size queries and
the argument refusals; and the oracle compiled by gcc, as oracle/ builds it,
linked with tests/sanitize/oracle_san.c, which runs every oracle entry point
on small inputs.  Any report aborts the program and fails the test.  The
library build takes about a minute on 8 cores; the test is skipped where the
compilers are missing."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_bit_wq_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "lib", "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not found")
def test_libwq_host_code_under_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    # Host side sanitized (each -fsanitize= after -Xarch_host); the device
    # code is compiled but never run.
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(f):
        out = str(tmp_path / (f[:-4] + ".o"))
        _run([HIPCC, "-std=c++17", "--offload-arch=gfx950", "-O1", "-g", "-fPIC",
              "-Xarch_device", "-O1", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + host_san +
             ["-c", os.path.join(CSRC, f), "-o", out])
        return out

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "host_san.o")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "host_san.c"), "-o", drv])
    exe = str(tmp_path / "host_san")
    _run([CLANGXX, "-fsanitize=address,undefined", "-o", exe, drv] + objs +
         ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    r = _run([exe], env=ENV, timeout=300)
    assert "host sanitizer run ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
          os.path.join(SAN, "oracle_san.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"), timeout=300)
    assert "oracle sanitizer run ok" in r.stdout
